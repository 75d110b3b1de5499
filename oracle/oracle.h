/*
 * oracle.h -- plain fp64 CPU reference for the batch-1 MoE verify hot path.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load this library. The GPU library shares no code, header,
 * table or constant with it, and neither side includes or links the other.
 *
 * Source of the method: the LMSYS post "Chasing the batch-1 floor:
 * Ling-3.0-flash speculative decode on Blackwell" (2026-08-21):
 *   - section "PDL: the latency floor of stacked small kernels", Fig. 7:
 *     router chain (gate matvec -> top-k) and MoE chain
 *     (up-GEMM -> activation -> down-GEMM -> combine);
 *   - section "Two fusions and a retune": SwiGLU silu(gate)*up computed in
 *     float; combine is an fp32 sum times the routing scale;
 *   - section "bf16 router gate and lm_head": both weights are bf16 and are
 *     pure bandwidth; the lm_head result feeds a greedy (argmax) verdict.
 *
 * Conventions shared by every function here:
 *   - bf16 tensors are raw uint16 bit patterns, row-major, reduction axis
 *     contiguous;
 *   - every sum is taken in double, over the reduction index in ascending
 *     order, with no blocking or reordering;
 *   - a selection (top-k, argmax) is decided on the logits rounded to fp32,
 *     the precision the post runs those logits in, lowest index first among
 *     equal fp32 values;
 *   - the functions return 0 on success and a negative code on bad
 *     arguments: -1 null pointer, -2 bad size, -3 index out of range,
 *     -4 non-finite input.
 */
#ifndef MOE_VERIFY_ORACLE_H
#define MOE_VERIFY_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exact value of one bf16 bit pattern (bf16 is the top half of an IEEE
 * binary32, so widening is exact). */
double oracle_bf16_value(uint16_t bits);

/* Router: logits, softmax top-k, renormalised weights.
 *   x      [M,H] bf16    token activations
 *   wg     [E,H] bf16    router gate weight
 *   bias   [E]   float   added to every token's logits, or NULL
 * outputs (all caller-owned):
 *   logits [M,E] double  l[t,e] = sum_h x[t,h]*wg[e,h] + bias[e]
 *   idx    [M,k] int32   k largest fp32-rounded logits, descending,
 *                        ties to the lower expert id
 *   w      [M,k] double  softmax restricted to the selected set
 *   w_full [M,k] double  softmax over all E experts, then renormalised
 *                        over the selected set (must equal w)
 *   gap_sel   [M] double l_(k) - l_(k+1) over the sorted fp64 logits
 *                        (+inf when k == E): a small gap means the set
 *                        boundary is a near-tie
 *   gap_order [M] double min_{j<k-1} l_(j) - l_(j+1): a small gap means the
 *                        order inside the set is a near-tie (+inf if k == 1)
 */
int oracle_route(const uint16_t *x, const uint16_t *wg, const float *bias,
                 int32_t M, int32_t H, int32_t E, int32_t k,
                 double *logits, int32_t *idx, double *w, double *w_full,
                 double *gap_sel, double *gap_order);

/* Selected experts' SwiGLU FFN and weighted combine.
 *   x      [M,H]    bf16
 *   idx    [M,k]    int32 expert ids (may repeat across tokens)
 *   w      [M,k]    double routing weights
 *   wgate  [E,I,H]  bf16, wup [E,I,H] bf16, wdown [E,H,I] bf16
 * output:
 *   out    [M,H] double
 *     out[t,r] = sum_j w[t,j] * sum_i wdown[e,r,i] * silu(g_i) * u_i,
 *     e = idx[t,j], g_i = wgate[e,i,:].x[t,:], u_i = wup[e,i,:].x[t,:],
 *     silu(z) = z / (1 + exp(-z)); slots summed in order j = 0..k-1.
 *   act    [M,k,I] double, optional (NULL skips): silu(g)*u per pair.
 */
int oracle_expert_ffn(const uint16_t *x, const int32_t *idx, const double *w,
                      const uint16_t *wgate, const uint16_t *wup,
                      const uint16_t *wdown,
                      int32_t M, int32_t H, int32_t I, int32_t E, int32_t k,
                      double *out, double *act);

/* lm_head projection and greedy argmax.
 *   h [M,H] bf16, wlm [V,H] bf16
 * outputs:
 *   tok  [M] int32  first v with the largest fp32-rounded z[t,v]
 *   zmax [M] double z[t,tok[t]] in fp64
 *   gap  [M] double z_(1) - z_(2) over the fp64 logits (+inf when V == 1)
 */
int oracle_lmhead(const uint16_t *h, const uint16_t *wlm,
                  int32_t M, int32_t H, int32_t V,
                  int32_t *tok, double *zmax, double *gap);

/* The norm at the head of the router chain (section "PDL: the latency floor
 * of stacked small kernels", Fig. 7: norm -> gate matvec -> top-k), read as
 * RMSNorm with a per-column gain and one rounding to bf16.
 *   h     [M,H] bf16  hidden states
 *   gamma [H]   bf16  gain
 *   eps         >= 0  added to the mean square
 * outputs:
 *   xn       [M,H] bf16 bits  the bf16 value nearest (ties to an even
 *                             significand) to
 *                             h[t,i] * gamma[i] / sqrt(mean_i h[t,i]^2 + eps)
 *   xn_exact [M,H] double     optional (NULL skips): that value in fp64
 * Returns -4 when a row's mean square plus eps is zero.
 */
int oracle_rmsnorm(const uint16_t *h, const uint16_t *gamma, double eps,
                   int32_t M, int32_t H, uint16_t *xn, double *xn_exact);

/* fp8 weights (the post's next bandwidth lever, section "The economics of
 * speculation at batch 1"), read as OCP E4M3 codes with one fp32 scale per
 * output row: W[row, j] = e4m3(q[row, j]) * scale[row].
 *
 * Value of one E4M3 byte: sign bit, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent 0 holds the subnormals m/8 * 2^-6; S.1111.111 is NaN;
 * there are no infinities (largest finite 448). */
double oracle_e4m3_value(uint8_t q);

/* oracle_expert_ffn with fp8 expert weights:
 *   qgate, qup [E,I,H] e4m3 with sgate, sup [E,I] fp32 (per row i),
 *   qdown [E,H,I] e4m3 with sdown [E,H] fp32 (per row r);
 * everything else as oracle_expert_ffn. NaN codes are rejected (-4). */
int oracle_expert_ffn_fp8(const uint16_t *x, const int32_t *idx, const double *w,
                          const uint8_t *qgate, const float *sgate,
                          const uint8_t *qup, const float *sup,
                          const uint8_t *qdown, const float *sdown,
                          int32_t M, int32_t H, int32_t I, int32_t E, int32_t k,
                          double *out);

/* oracle_lmhead with an fp8 lm_head: qlm [V,H] e4m3, slm [V] fp32. */
int oracle_lmhead_fp8(const uint16_t *h, const uint8_t *qlm, const float *slm,
                      int32_t M, int32_t H, int32_t V,
                      int32_t *tok, double *zmax, double *gap);

/* Greedy verdict of one verify step over a drafted chain (section "The
 * shape of a single-request step": the target scores the whole chain in one
 * forward and the verdict is taken inside the verify step).
 *   tokens [M] int32  the chain the target scored: tokens[0] is the root
 *                     (committed by the previous step), tokens[1..M-1] the
 *                     drafted candidates in chain order
 *   tok    [M] int32  the target's greedy token after each chain position
 *                     (tok of oracle_lmhead)
 * output:
 *   accept [2] int32  accept[0] = n + 1, n = the number of leading drafted
 *                     candidates equal to the target's token at the position
 *                     before them (tokens[i] == tok[i-1], i = 1..n; the
 *                     first mismatch ends the prefix); accept[1] = tok[n],
 *                     the bonus token and next root.
 * The step commits tok[0..n]: the n accepted candidates and the bonus token.
 */
int oracle_greedy_verdict(const int32_t *tokens, const int32_t *tok, int32_t M,
                          int32_t *accept);

/* Thread count of the OpenMP loops (n >= 1), and the current count. */
void oracle_set_threads(int32_t n);
int32_t oracle_threads(void);

#ifdef __cplusplus
}
#endif

#endif
