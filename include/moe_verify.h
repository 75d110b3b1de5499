/*
 * moe_verify.h -- C ABI of the MI355X (gfx950) batch-1 MoE verify hot path.
 *
 * The path is the weight-bandwidth-bound part of one speculative-decode
 * verify step of a 512-expert MoE model, as the LMSYS post "Chasing the
 * batch-1 floor: Ling-3.0-flash speculative decode on Blackwell" describes
 * it:
 *   - router chain: gate matvec then top-k (section "PDL: the latency floor
 *     of stacked small kernels", Fig. 7), gate weight in bf16 (section
 *     "bf16 router gate and lm_head");
 *   - MoE chain: expert grouping, up projection with SwiGLU folded into it,
 *     down projection and an fp32 weighted combine (section "Two fusions and
 *     a retune");
 *   - lm_head projection in bf16 feeding the greedy verdict (section "bf16
 *     router gate and lm_head"; the verdict itself, section "The shape of a
 *     single-request step", Fig. 3).
 *
 * Conventions (every entry point):
 *   - All tensor pointers are DEVICE pointers owned by the caller. The
 *     library never allocates, frees, copies to the host or synchronises.
 *   - bf16 tensors are raw uint16 bit patterns; every matrix is row-major
 *     with the reduction axis contiguous.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = legacy default
 *     stream) and runs asynchronously. A device fault surfaces at the
 *     caller's next synchronisation.
 *   - Device values (expert ids, routing weights) are never read on the
 *     host: one call can consume what the previous call on the same stream
 *     produced.
 *   - The status is MOE_OK when the work was enqueued. Errors come from
 *     host-side argument checks (nothing is launched then) or from the
 *     launch itself (MOE_ERR_LAUNCH).
 *   - Pointers to bf16/fp32 tensors must be 16-byte aligned (128-bit
 *     loads). Shape limits: 1 <= M <= 16, 1 <= k <= min(E, 16),
 *     1 <= E <= 1024, H and I multiples of 8 and at most 8192,
 *     1 <= V < 2^31.
 *   - Wider rows: the kernels keep every token's row of the hidden
 *     dimension on chip (the expert up kernel and the lm_head stage the M
 *     rows of x or h in LDS, 160 KB per CU; the norm holds each lane's
 *     share in registers), so above some H a call is refused with
 *     MOE_ERR_UNSUPPORTED before anything is launched. The largest H
 *     accepted, by M (every smaller multiple of 8, or of 16 for fp8
 *     weights, is accepted; the limit depends on M and H only, not on I,
 *     E, k or V):
 *
 *        M   experts bf16   experts fp8   lm_head bf16   lm_head fp8   norm
 *       1-5      8192           8192          8192           8192       8192
 *        6       8192           8192          7936           7680       8192
 *        7       8192           8192          6656           6656       8192
 *        8       8192           8192          5888           5632       8192
 *        9       6144           5120          5120           5120       4096
 *       10       6144           5120          4608           4608       4096
 *       11       6144           5120          4352           4096       4096
 *       12       4096           5120          3840           3584       4096
 *       13       4096           5120          3584           3584       4096
 *       14       4096           5120          3328           3072       4096
 *       15       4096           4096          3072           3072       4096
 *       16       4096           4096          2816           2560       4096
 *
 *     "experts" covers moe_expert_ffn, moe_expert_ffn_shared and the
 *     moe_layer entry points (with their fp8 variants), "lm_head" the
 *     lmhead_* entry points, "norm" moe_route_rmsnorm and
 *     moe_layer_rmsnorm (which also takes the experts' limit). The model's
 *     width, H = 2560, is accepted everywhere at every M.
 *   - Workspaces: size from the matching *_workspace_bytes query,
 *     16-byte aligned, ZERO-FILLED before their first use (one
 *     moe_workspace_clear call, or any zero fill). The first 4096 bytes of
 *     every workspace are a header whose counters (arrival tickets, one per
 *     128-byte line) sit at fixed offsets; every call leaves them at zero
 *     again, so one workspace is reused by every entry point and shape
 *     without clearing.
 *     Two calls that may run concurrently must not share a workspace.
 *   - Results are deterministic: no floating-point atomics; rerunning a
 *     call on the same inputs gives bitwise-equal outputs. A token's results
 *     do not depend on the other tokens in the call as long as M stays on
 *     the same side of two regime limits: the router sums a logit over
 *     8-row tiles for M <= 8 and 16-row tiles above, and the down
 *     projection takes its matrix-core kernel once the pairs' activations
 *     (M*k*I*2 bytes) pass 150 KB. With fp8 weights a third: an expert that
 *     serves at least 4 of the call's (token, slot) pairs runs its up
 *     projection on the matrix cores. Across a limit the sums run in
 *     another order and agree within rounding.
 */
#ifndef MOE_VERIFY_H
#define MOE_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status_t;

enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL */
    MOE_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
    MOE_ERR_UNSUPPORTED = 3, /* a size this library does not handle */
    MOE_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
    MOE_ERR_WORKSPACE = 5,   /* workspace smaller than its query */
    MOE_ERR_LAUNCH = 6       /* the kernel launch failed */
};

/* ABI version; bumps on any signature or semantic change. */
int32_t moe_abi_version(void);

/* Static string naming a status (never NULL). */
const char *moe_status_str(moe_status_t status);

/* Zero-fill a workspace on `stream` with a fill kernel (capturable in a
 * graph). bytes must be a multiple of 16. */
moe_status_t moe_workspace_clear(void *workspace, size_t bytes, void *stream);

/* ------------------------------------------------------------------------
 * moe_hbm_read_probe -- a plain streaming read of `bytes` of device memory,
 * the measured HBM read ceiling against which the kernels' rates are set
 * (cold-weight bandwidth is the bound of every step of the path).
 * MOE_HBM_PROBE_GROUPS workgroups of 256 threads read 16-byte chunks in
 * grid-stride order (chunk c by thread c mod 65536) with non-temporal
 * loads, eight in flight per thread, and fold every 32-bit word into an
 * XOR.
 *
 *   src        device memory, 16-byte aligned, bytes a positive multiple
 *              of 16; only read
 *   checksums  [MOE_HBM_PROBE_GROUPS] u32 out: the XOR of the words each
 *              workgroup read (their XOR is the XOR of all words of src)
 *
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (bytes), MOE_ERR_ALIGN.
 * ---------------------------------------------------------------------- */
#define MOE_HBM_PROBE_GROUPS 256
moe_status_t moe_hbm_read_probe(const void *src, size_t bytes, uint32_t *checksums,
                                void *stream);

/* ------------------------------------------------------------------------
 * moe_route -- router gate GEMV, softmax top-k, renormalised weights.
 * (router chain: gate matvec -> top-k; section "PDL: the latency floor of
 *  stacked small kernels", Fig. 7; bf16 gate, section "bf16 router gate
 *  and lm_head")
 *
 *   x         [M,H] bf16   token activations
 *   w_router  [E,H] bf16   gate weight
 *   bias      [E]   fp32   added to every logit before selection and
 *                          softmax, or NULL for none
 *   topk_idx  [M,k] int32  out: the k experts with the largest fp32 logits,
 *                          in descending logit order, ties to the lower id
 *   topk_w    [M,k] fp32   out: softmax of the selected logits (equal to a
 *                          softmax over all E renormalised over the set)
 *   logits    [M,E] fp32   optional out (NULL skips): l = x.w_router^T + bias
 *   workspace              moe_route_workspace_bytes(M, E) bytes: the
 *                          counter header and the partial logits
 *                          [slices][M][E] fp32 of the workgroups that split
 *                          the hidden dimension (up to four slices, so a
 *                          2.6 MB gate spreads over every CU); the last
 *                          workgroup to arrive sums them in slice order and
 *                          selects. Its size depends on M and E only.
 *
 * Errors: MOE_ERR_NULL (x, w_router, topk_idx, topk_w or workspace NULL),
 * MOE_ERR_SHAPE (M, H, E or k below 1), MOE_ERR_UNSUPPORTED (the shape
 * limits above), MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH.
 * ---------------------------------------------------------------------- */
size_t moe_route_workspace_bytes(int32_t M, int32_t E);
moe_status_t moe_route(const uint16_t *x, const uint16_t *w_router,
                       const float *bias, int32_t M, int32_t H, int32_t E,
                       int32_t k, int32_t *topk_idx, float *topk_w,
                       float *logits, void *workspace, size_t workspace_bytes,
                       void *stream);

/* ------------------------------------------------------------------------
 * moe_route_rmsnorm -- the router chain with its norm in front: RMSNorm,
 * then moe_route on the normalised rows, in one launch. (Router chain
 * norm -> gate matvec -> top-k, section "PDL: the latency floor of stacked
 * small kernels", Fig. 7; the norm is read as RMSNorm with a per-column
 * gain, rounded once to bf16.)
 *
 *   h         [M,H] bf16   hidden states before the norm
 *   gamma     [H]   bf16   gain (16-byte aligned)
 *   eps              fp32  added to each row's mean square (>= 0, finite)
 *   x_norm    [M,H] bf16   out: the bf16 value nearest to
 *                          h[t,i] * gamma[i] / sqrt(mean_i h[t,i]^2 + eps)
 *                          (ties to even); the gate reads exactly these
 *                          values, and moe_expert_ffn should too
 *   w_router, bias, M, H, E, k, topk_idx, topk_w, logits, workspace:
 *                          as moe_route (same workspace size)
 *
 * Errors: as moe_route; MOE_ERR_NULL for a NULL gamma or x_norm,
 * MOE_ERR_SHAPE for a negative, NaN or infinite eps, MOE_ERR_ALIGN unless
 * gamma and x_norm are 16-byte aligned, MOE_ERR_UNSUPPORTED when M > 8 and
 * H > 4096 (every hidden-state chunk of a lane must fit in registers; the
 * "norm" column of the limits table).
 * ---------------------------------------------------------------------- */
moe_status_t moe_route_rmsnorm(const uint16_t *h, const uint16_t *gamma, float eps,
                               const uint16_t *w_router, const float *bias,
                               int32_t M, int32_t H, int32_t E, int32_t k,
                               uint16_t *x_norm, int32_t *topk_idx, float *topk_w,
                               float *logits, void *workspace,
                               size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * moe_expert_ffn -- selected experts' SwiGLU FFN with weighted combine.
 * (MoE chain: grouping -> up-GEMM with SwiGLU epilogue -> down-GEMM ->
 *  combine; section "Two fusions and a retune")
 *
 *   x         [M,H]   bf16   token activations
 *   topk_idx  [M,k]   int32  expert of each (token, slot) pair; ids may
 *                            repeat across tokens; an id outside [0,E)
 *                            makes the pair contribute nothing
 *   topk_w    [M,k]   fp32   routing weight of each pair
 *   w_gate    [E,I,H] bf16   gate projection rows
 *   w_up      [E,I,H] bf16   up projection rows
 *   w_down    [E,H,I] bf16   down projection rows
 *   out       [M,H]   fp32   out (overwritten):
 *       out[t,:] = sum_{j<k} topk_w[t,j] * W_down[e] (silu(W_gate[e] x_t)
 *                  * (W_up[e] x_t)),  e = topk_idx[t,j],
 *       silu(z) = z / (1 + exp(-z)) in fp32, the SwiGLU product rounded once
 *       to bf16 before the down projection, slots summed in order in fp32.
 *   workspace                moe_expert_ffn_workspace_bytes(M,H,I,E,k) bytes
 *
 * Every distinct selected expert's weights are read from HBM exactly once
 * per call, however many tokens chose it.
 *
 * Errors: MOE_ERR_NULL (any tensor or the workspace NULL), MOE_ERR_SHAPE
 * (M, H, I, E or k below 1), MOE_ERR_UNSUPPORTED (I not a multiple of 8 or
 * above 8192, or the "experts bf16" limit of the table above),
 * MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH.
 * ---------------------------------------------------------------------- */
size_t moe_expert_ffn_workspace_bytes(int32_t M, int32_t H, int32_t I,
                                      int32_t E, int32_t k);
moe_status_t moe_expert_ffn(const uint16_t *x, const int32_t *topk_idx,
                            const float *topk_w, const uint16_t *w_gate,
                            const uint16_t *w_up, const uint16_t *w_down,
                            int32_t M, int32_t H, int32_t I, int32_t E,
                            int32_t k, float *out, void *workspace,
                            size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * moe_expert_ffn_shared -- moe_expert_ffn plus one shared expert that every
 * token uses with weight 1, streamed in the same launches as one more bucket
 * of the grouping (the "513-expert" MoE decode of section "Two fusions and a
 * retune": 512 routed experts and one more). The shared expert's form is a
 * reading: a SwiGLU FFN of the routed experts' shape, no gate on its output.
 *
 *   x, topk_idx, topk_w, w_gate, w_up, w_down, M, H, I, E, k, workspace:
 *                           as moe_expert_ffn (same workspace size)
 *   w_gate_shared [I,H] bf16, w_up_shared [I,H] bf16, w_down_shared [H,I]
 *                           bf16: the shared expert (16-byte aligned)
 *   out      [M,H]   fp32   out (overwritten): moe_expert_ffn's sum over the
 *                           k slots in order, then + the shared expert's
 *                           W_down_s (silu(W_gate_s x_t) * (W_up_s x_t)),
 *                           same rounding rules
 * Errors: as moe_expert_ffn; MOE_ERR_NULL for a NULL shared tensor,
 * MOE_ERR_ALIGN for a misaligned one, MOE_ERR_UNSUPPORTED when
 * M * (k + 1) > 256 or E > 1023.
 * ---------------------------------------------------------------------- */
moe_status_t moe_expert_ffn_shared(const uint16_t *x, const int32_t *topk_idx,
                                   const float *topk_w, const uint16_t *w_gate,
                                   const uint16_t *w_up, const uint16_t *w_down,
                                   const uint16_t *w_gate_shared,
                                   const uint16_t *w_up_shared,
                                   const uint16_t *w_down_shared, int32_t M,
                                   int32_t H, int32_t I, int32_t E, int32_t k,
                                   float *out, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * moe_expert_ffn_fp8 -- moe_expert_ffn with fp8 expert weights: the post's
 * next bandwidth lever (section "The economics of speculation at batch 1"),
 * read as OCP E4M3 codes with one fp32 scale per output row, which halves
 * the bytes every selected expert streams.
 *
 *   w_gate, w_up [E,I,H] uint8   E4M3 codes (16-byte aligned)
 *   s_gate, s_up [E,I]   fp32    row scales: W_gate[e,i,h] =
 *                                s_gate[e,i] * e4m3(w_gate[e,i,h])
 *   w_down       [E,H,I] uint8   E4M3 codes
 *   s_down       [E,H]   fp32    row scales of W_down
 *   the rest:                    as moe_expert_ffn (same workspace size)
 * H and I must be multiples of 16 (else MOE_ERR_UNSUPPORTED), and H within
 * the "experts fp8" column of the limits table above. NaN codes are the
 * caller's to avoid.
 * ---------------------------------------------------------------------- */
moe_status_t moe_expert_ffn_fp8(const uint16_t *x, const int32_t *topk_idx,
                                const float *topk_w, const uint8_t *w_gate,
                                const float *s_gate, const uint8_t *w_up,
                                const float *s_up, const uint8_t *w_down,
                                const float *s_down, int32_t M, int32_t H,
                                int32_t I, int32_t E, int32_t k, float *out,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

/* ------------------------------------------------------------------------
 * moe_layer -- one MoE layer verify step: moe_route then moe_expert_ffn,
 * enqueued back to back on `stream` (same arguments and results as the two
 * calls; topk_idx/topk_w are written and then consumed on the device).
 *   workspace  moe_layer_workspace_bytes(M,H,I,E,k) bytes
 * ---------------------------------------------------------------------- */
size_t moe_layer_workspace_bytes(int32_t M, int32_t H, int32_t I, int32_t E,
                                 int32_t k);
moe_status_t moe_layer(const uint16_t *x, const uint16_t *w_router,
                       const float *bias, const uint16_t *w_gate,
                       const uint16_t *w_up, const uint16_t *w_down,
                       int32_t M, int32_t H, int32_t I, int32_t E, int32_t k,
                       int32_t *topk_idx, float *topk_w, float *out,
                       void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * moe_layer_noalloc -- moe_layer without a caller workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). The same kernels run with
 * their scratch (arrival counters, partial router logits, the pairs'
 * activations) in a library-owned array of MOE_NOALLOC_SCRATCH_BYTES that
 * every GPU the library runs on holds, one copy per device, until the
 * process ends. The call itself allocates nothing: at its first call on a
 * device it looks the array's device address up and clears its counter
 * header with a fill kernel on `stream`; every call leaves the counters at
 * zero again, as with a workspace.
 *
 *   Arguments and results: as moe_layer, without workspace/workspace_bytes.
 *
 * Every call on one GPU shares that GPU's array and it keeps the last call's
 * contents: calls that may overlap on one GPU (two streams, two host
 * threads) race and must be serialised by the caller. Errors: as moe_layer;
 * MOE_ERR_WORKSPACE when moe_layer_workspace_bytes(M,H,I,E,k) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES (never for the shapes moe_layer admits: the
 * largest needs 4,722,688 bytes), MOE_ERR_LAUNCH when the array's address
 * cannot be found on the current device.
 * ---------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)5 << 20)
moe_status_t moe_layer_noalloc(const uint16_t *x, const uint16_t *w_router,
                               const float *bias, const uint16_t *w_gate,
                               const uint16_t *w_up, const uint16_t *w_down,
                               int32_t M, int32_t H, int32_t I, int32_t E,
                               int32_t k, int32_t *topk_idx, float *topk_w,
                               float *out, void *stream);

/* ------------------------------------------------------------------------
 * moe_layer_shared -- moe_route then moe_expert_ffn_shared on one stream.
 *   Arguments as moe_layer, plus the shared expert's three tensors as in
 *   moe_expert_ffn_shared. Workspace: moe_layer_workspace_bytes.
 * ---------------------------------------------------------------------- */
moe_status_t moe_layer_shared(const uint16_t *x, const uint16_t *w_router,
                              const float *bias, const uint16_t *w_gate,
                              const uint16_t *w_up, const uint16_t *w_down,
                              const uint16_t *w_gate_shared,
                              const uint16_t *w_up_shared,
                              const uint16_t *w_down_shared, int32_t M, int32_t H,
                              int32_t I, int32_t E, int32_t k, int32_t *topk_idx,
                              float *topk_w, float *out, void *workspace,
                              size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * moe_layer_fp8 -- moe_route (bf16 gate) then moe_expert_ffn_fp8, on one
 * stream. Arguments as moe_layer with the fp8 expert tensors and scales of
 * moe_expert_ffn_fp8. Workspace: moe_layer_workspace_bytes.
 * ---------------------------------------------------------------------- */
moe_status_t moe_layer_fp8(const uint16_t *x, const uint16_t *w_router,
                           const float *bias, const uint8_t *w_gate,
                           const float *s_gate, const uint8_t *w_up,
                           const float *s_up, const uint8_t *w_down,
                           const float *s_down, int32_t M, int32_t H, int32_t I,
                           int32_t E, int32_t k, int32_t *topk_idx, float *topk_w,
                           float *out, void *workspace, size_t workspace_bytes,
                           void *stream);

/* ------------------------------------------------------------------------
 * moe_layer_rmsnorm -- moe_route_rmsnorm then moe_expert_ffn on the
 * normalised rows it wrote (x_norm), on one stream: the whole router chain
 * (norm -> gate -> top-k) and MoE chain of the section "PDL: the latency
 * floor of stacked small kernels", Fig. 7.
 *
 *   h, gamma, eps, x_norm:  as moe_route_rmsnorm
 *   the rest:               as moe_layer (same workspace size)
 * Errors: those of moe_route_rmsnorm and moe_expert_ffn.
 * ---------------------------------------------------------------------- */
moe_status_t moe_layer_rmsnorm(const uint16_t *h, const uint16_t *gamma, float eps,
                               const uint16_t *w_router, const float *bias,
                               const uint16_t *w_gate, const uint16_t *w_up,
                               const uint16_t *w_down, int32_t M, int32_t H,
                               int32_t I, int32_t E, int32_t k, uint16_t *x_norm,
                               int32_t *topk_idx, float *topk_w, float *out,
                               void *workspace, size_t workspace_bytes,
                               void *stream);

/* ------------------------------------------------------------------------
 * lmhead_argmax -- lm_head GEMV fused with the greedy argmax.
 * (bf16 lm_head, section "bf16 router gate and lm_head"; greedy decoding,
 *  section "The shape of a single-request step")
 *
 *   h          [M,H] bf16   final hidden states
 *   w_lm       [V,H] bf16   lm_head rows
 *   argmax     [M]   int32  out: first v with the largest fp32 logit
 *                           z[t,v] = h[t,:].w_lm[v,:] (lowest id on ties)
 *   max_logit  [M]   fp32   optional out (NULL skips): z[t, argmax[t]]
 *   workspace               lmhead_argmax_workspace_bytes(M, V) bytes: the
 *                           counter header and one M-key slot per workgroup
 *                           (each workgroup's per-token winner, merged by
 *                           a second one-workgroup kernel that the call
 *                           enqueues behind the first on `stream`). V is
 *                           an argument because
 *                           the workgroup count is min(ceil(V/16), 256):
 *                           the query returns 0 for an invalid M or V, and
 *                           today's size is that of 256 workgroups.
 *
 * The [M,V] logits are never written to memory. A NaN logit counts as
 * -inf; when every logit of a row is -inf (or NaN) the row's argmax is 0.
 *
 * Errors: MOE_ERR_NULL (h, w_lm, argmax or workspace NULL), MOE_ERR_SHAPE
 * (M, H or V below 1), MOE_ERR_UNSUPPORTED (M above 16, H not a multiple of
 * 8 or above the "lm_head bf16" limit of the table above), MOE_ERR_ALIGN,
 * MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH.
 * ---------------------------------------------------------------------- */
size_t lmhead_argmax_workspace_bytes(int32_t M, int32_t V);
moe_status_t lmhead_argmax(const uint16_t *h, const uint16_t *w_lm,
                           int32_t M, int32_t H, int32_t V, int32_t *argmax,
                           float *max_logit, void *workspace,
                           size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * lmhead_greedy_verify -- lmhead_argmax and, in the same call, the greedy
 * verdict of the verify chain. (Section "The shape of a single-request
 * step": the target scores the drafted chain in one forward and the verdict
 * is taken inside the verify step, on the device; greedy decoding.)
 *
 *   h, w_lm, M, H, V, argmax, max_logit, workspace: as lmhead_argmax; row t
 *              of h is the target's hidden state at chain position t
 *   tokens     [M] int32  the chain the target scored: tokens[0] the root
 *                         (committed by the previous step), tokens[1..M-1]
 *                         the drafted candidates in chain order
 *   accept     [2] int32  out: accept[0] = n + 1, where n counts the leading
 *                         candidates with tokens[i] == argmax[i-1]
 *                         (i = 1..n; the first mismatch ends the prefix);
 *                         accept[1] = argmax[n], the bonus token and the
 *                         next step's root
 *
 * The step commits argmax[0..n] (n accepted candidates, then the bonus
 * token). tokens is read on the device only; any int32 value is allowed.
 * Errors: as lmhead_argmax; MOE_ERR_NULL if tokens or accept is NULL,
 * MOE_ERR_ALIGN unless both are 4-byte aligned. Uses the same workspace
 * size as lmhead_argmax.
 * ---------------------------------------------------------------------- */
moe_status_t lmhead_greedy_verify(const uint16_t *h, const uint16_t *w_lm,
                                  const int32_t *tokens, int32_t M, int32_t H,
                                  int32_t V, int32_t *argmax, float *max_logit,
                                  int32_t *accept, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * lmhead_argmax_fp8, lmhead_greedy_verify_fp8 -- the same with an fp8
 * lm_head: the post's next bandwidth lever ("once fp8 weights shrink the
 * fixed base", section "The economics of speculation at batch 1"), read as
 * OCP E4M3 codes with one fp32 scale per vocabulary row.
 *
 *   w_lm     [V,H] uint8  E4M3 codes (sign, 4 exponent bits with bias 7,
 *                         3 mantissa bits; S.1111.111 is NaN), 16-byte aligned
 *   w_scale  [V]   fp32   z[t,v] = w_scale[v] * sum_h h[t,h] * e4m3(w_lm[v,h])
 *   the rest: as lmhead_argmax / lmhead_greedy_verify (same workspace size)
 * H must be a multiple of 16. NaN codes are the caller's to avoid (the
 * argmax over a NaN logit is unspecified).
 * ---------------------------------------------------------------------- */
moe_status_t lmhead_argmax_fp8(const uint16_t *h, const uint8_t *w_lm,
                               const float *w_scale, int32_t M, int32_t H,
                               int32_t V, int32_t *argmax, float *max_logit,
                               void *workspace, size_t workspace_bytes,
                               void *stream);
moe_status_t lmhead_greedy_verify_fp8(const uint16_t *h, const uint8_t *w_lm,
                                      const float *w_scale, const int32_t *tokens,
                                      int32_t M, int32_t H, int32_t V,
                                      int32_t *argmax, float *max_logit,
                                      int32_t *accept, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * lmhead_partial_keys, lmhead_partial_keys_fp8, lmhead_merge_keys -- the two
 * phases that lmhead_argmax and lmhead_greedy_verify (and their fp8
 * variants) enqueue, as separate calls, for callers that time the
 * lm_head's GEMV alone or put other work between the phases. (Same
 * sections as lmhead_argmax.)
 *
 * lmhead_partial_keys(_fp8): the GEMV. Arguments as lmhead_argmax(_fp8)
 *   without the outputs; every workgroup writes its per-token winner (a
 *   64-bit key: the logit's order code, then the row) into the workspace.
 * lmhead_merge_keys: the merge of those keys, then the verdict when tokens
 *   is given. argmax, max_logit (optional), tokens and accept as in
 *   lmhead_greedy_verify; tokens and accept both NULL for lmhead_argmax's
 *   outputs alone. workspace: the one the partial-keys call wrote, with the
 *   same M and V, on the same stream after it (nothing may write the
 *   workspace in between).
 *
 * partial keys then merge keys gives bitwise the outputs of the combined
 * call. Errors: those of lmhead_argmax(_fp8) for their arguments;
 * lmhead_merge_keys: MOE_ERR_NULL (argmax or workspace NULL, or only one
 * of tokens and accept given), MOE_ERR_SHAPE (M or V below 1),
 * MOE_ERR_UNSUPPORTED (M above 16), MOE_ERR_ALIGN, MOE_ERR_WORKSPACE,
 * MOE_ERR_LAUNCH.
 * ---------------------------------------------------------------------- */
moe_status_t lmhead_partial_keys(const uint16_t *h, const uint16_t *w_lm, int32_t M,
                                 int32_t H, int32_t V, void *workspace,
                                 size_t workspace_bytes, void *stream);
moe_status_t lmhead_partial_keys_fp8(const uint16_t *h, const uint8_t *w_lm,
                                     const float *w_scale, int32_t M, int32_t H,
                                     int32_t V, void *workspace, size_t workspace_bytes,
                                     void *stream);
moe_status_t lmhead_merge_keys(int32_t M, int32_t V, int32_t *argmax, float *max_logit,
                               const int32_t *tokens, int32_t *accept,
                               const void *workspace, size_t workspace_bytes,
                               void *stream);

#ifdef __cplusplus
}
#endif

#endif
