/*
 * oracle.c -- plain fp64 CPU reference for the batch-1 MoE verify hot path.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load this library; the GPU library never does. Every
 * function is the plain definition of what the step computes, written from
 * the LMSYS post "Chasing the batch-1 floor: Ling-3.0-flash speculative
 * decode on Blackwell": double-precision sums in ascending index order, no
 * blocking, no fusion. OpenMP only splits independent outputs between
 * threads; it never changes the order of any sum.
 *
 * Readings of points the post leaves open (each is listed with its reason
 * in the design notes):
 *   - scoring is a softmax over the router logits, k = 8 in the model, and
 *     the k weights are renormalised over the selected set;
 *   - the optional router bias is added to the logits before both the
 *     selection and the softmax;
 *   - selection and argmax are decided on fp32-rounded logits (the post runs
 *     fp32 logits), ties to the lower index;
 *   - silu(z) = z / (1 + exp(-z)), applied to the gate projection and
 *     multiplied by the up projection (section "Two fusions and a retune");
 *   - the combine sums the k slots in slot order (same section);
 *   - fp8 weights are OCP E4M3 codes times one fp32 scale per output row;
 *   - the router chain's norm is RMSNorm with a per-column gain, rounded
 *     once to bf16 (the value both the gate and the experts read);
 *   - the verify chain is scored greedily: a drafted candidate is accepted
 *     while it equals the target's argmax at the position before it, and
 *     the target's argmax after the last accepted position is the bonus
 *     token (section "The shape of a single-request step", greedy decoding
 *     throughout).
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* Threads the OpenMP loops below use from now on (n >= 1), and how many
 * they use: set once for a single-threaded timing, once for all cores.
 * Thread counts never change a result, only which thread computes it. */
void oracle_set_threads(int32_t n)
{
    if (n >= 1)
        omp_set_num_threads(n);
}

int32_t oracle_threads(void)
{
    return (int32_t)omp_get_max_threads();
}

double oracle_bf16_value(uint16_t bits)
{
    /* bf16 is the upper 16 bits of a binary32 value. */
    uint32_t wide = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &wide, sizeof f);
    return (double)f;
}

/* Dot product of two bf16 rows of length n, in double, ascending index. */
static double dot_bf16(const uint16_t *a, const uint16_t *b, int64_t n)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i)
        s += oracle_bf16_value(a[i]) * oracle_bf16_value(b[i]);
    return s;
}

/* Dot product of a bf16 row with a double vector, ascending index. */
static double dot_bf16_f64(const uint16_t *a, const double *b, int64_t n)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i)
        s += oracle_bf16_value(a[i]) * b[i];
    return s;
}

static int all_finite_bf16(const uint16_t *a, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if ((a[i] & 0x7F80u) == 0x7F80u) /* exponent all ones: inf or nan */
            return 0;
    return 1;
}

static int cmp_desc(const void *pa, const void *pb)
{
    double a = *(const double *)pa, b = *(const double *)pb;
    return (a < b) - (a > b);
}

/* Largest minus second-largest gap information over n values. */
static void sorted_gaps(const double *v, int32_t n, int32_t k,
                        double *gap_sel, double *gap_order)
{
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    memcpy(s, v, sizeof(double) * (size_t)n);
    qsort(s, (size_t)n, sizeof(double), cmp_desc);
    *gap_sel = (k < n) ? s[k - 1] - s[k] : INFINITY;
    double g = INFINITY;
    for (int32_t j = 0; j + 1 < k; ++j)
        if (s[j] - s[j + 1] < g)
            g = s[j] - s[j + 1];
    *gap_order = g;
    free(s);
}

int oracle_route(const uint16_t *x, const uint16_t *wg, const float *bias,
                 int32_t M, int32_t H, int32_t E, int32_t k,
                 double *logits, int32_t *idx, double *w, double *w_full,
                 double *gap_sel, double *gap_order)
{
    if (!x || !wg || !logits || !idx || !w || !w_full || !gap_sel || !gap_order)
        return -1;
    if (M < 1 || H < 1 || E < 1 || k < 1 || k > E)
        return -2;
    if (!all_finite_bf16(x, (int64_t)M * H) || !all_finite_bf16(wg, (int64_t)E * H))
        return -4;
    if (bias)
        for (int32_t e = 0; e < E; ++e)
            if (!isfinite(bias[e]))
                return -4;

    char *taken = (char *)malloc((size_t)E);
    double *p = (double *)malloc(sizeof(double) * (size_t)E);

    for (int32_t t = 0; t < M; ++t) {
        double *l = logits + (int64_t)t * E;

        /* Gate matvec (router chain, Fig. 7), plus the optional bias. */
        for (int32_t e = 0; e < E; ++e) {
            l[e] = dot_bf16(x + (int64_t)t * H, wg + (int64_t)e * H, H);
            if (bias)
                l[e] += (double)bias[e];
        }

        /* Top-k: k rounds, each picking the largest fp32-rounded logit not
         * yet taken; a strict comparison keeps the lower id on ties. */
        memset(taken, 0, (size_t)E);
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            float best_v = 0.0f;
            for (int32_t e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                float v = (float)l[e];
                if (best < 0 || v > best_v) {
                    best = e;
                    best_v = v;
                }
            }
            taken[best] = 1;
            idx[(int64_t)t * k + j] = best;
        }

        /* Softmax restricted to the selected set, shifted by its largest
         * member for range safety (the shift cancels in the ratio). */
        double m = l[idx[(int64_t)t * k]];
        double den = 0.0;
        for (int32_t j = 0; j < k; ++j)
            den += exp(l[idx[(int64_t)t * k + j]] - m);
        for (int32_t j = 0; j < k; ++j)
            w[(int64_t)t * k + j] = exp(l[idx[(int64_t)t * k + j]] - m) / den;

        /* Same weights the long way: softmax over all E experts, then
         * renormalised over the selected set. */
        double mx = l[0];
        for (int32_t e = 1; e < E; ++e)
            if (l[e] > mx)
                mx = l[e];
        double z = 0.0;
        for (int32_t e = 0; e < E; ++e) {
            p[e] = exp(l[e] - mx);
            z += p[e];
        }
        for (int32_t e = 0; e < E; ++e)
            p[e] /= z;
        double ps = 0.0;
        for (int32_t j = 0; j < k; ++j)
            ps += p[idx[(int64_t)t * k + j]];
        for (int32_t j = 0; j < k; ++j)
            w_full[(int64_t)t * k + j] = p[idx[(int64_t)t * k + j]] / ps;

        sorted_gaps(l, E, k, &gap_sel[t], &gap_order[t]);
    }
    free(taken);
    free(p);
    return 0;
}

/* SwiGLU of one row: silu on the gate projection, times the up projection
 * (section "Two fusions and a retune"), in double. */
static double swiglu(double g, double u)
{
    double s = g / (1.0 + exp(-g));
    return s * u;
}

int oracle_expert_ffn(const uint16_t *x, const int32_t *idx, const double *w,
                      const uint16_t *wgate, const uint16_t *wup,
                      const uint16_t *wdown,
                      int32_t M, int32_t H, int32_t I, int32_t E, int32_t k,
                      double *out, double *act)
{
    if (!x || !idx || !w || !wgate || !wup || !wdown || !out)
        return -1;
    if (M < 1 || H < 1 || I < 1 || E < 1 || k < 1)
        return -2;
    const int64_t NP = (int64_t)M * k;
    for (int64_t p = 0; p < NP; ++p)
        if (idx[p] < 0 || idx[p] >= E)
            return -3;
    if (!all_finite_bf16(x, (int64_t)M * H))
        return -4;
    for (int64_t p = 0; p < NP; ++p) {
        int64_t e = idx[p];
        if (!isfinite(w[p]) ||
            !all_finite_bf16(wgate + e * I * H, (int64_t)I * H) ||
            !all_finite_bf16(wup + e * I * H, (int64_t)I * H) ||
            !all_finite_bf16(wdown + e * H * I, (int64_t)H * I))
            return -4;
    }

    double *a = (double *)malloc(sizeof(double) * (size_t)(NP * I));
    double *y = (double *)malloc(sizeof(double) * (size_t)(NP * H));

    /* Up projection and SwiGLU for every (token, slot) pair: gate and up are
     * separate dot products, silu is taken on the gate, and the product is
     * kept in double (section "Two fusions and a retune"). */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t p = 0; p < NP; ++p)
        for (int32_t i = 0; i < I; ++i) {
            int32_t t = (int32_t)(p / k);
            int64_t e = idx[p];
            const uint16_t *xt = x + (int64_t)t * H;
            double g = dot_bf16(wgate + (e * I + i) * H, xt, H);
            double u = dot_bf16(wup + (e * I + i) * H, xt, H);
            a[p * I + i] = swiglu(g, u);
        }

    /* Down projection of every pair. */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t p = 0; p < NP; ++p)
        for (int32_t r = 0; r < H; ++r) {
            int64_t e = idx[p];
            y[p * H + r] = dot_bf16_f64(wdown + (e * H + r) * I, a + p * I, I);
        }

    /* Weighted combine, slots in order. */
    for (int32_t t = 0; t < M; ++t)
        for (int32_t r = 0; r < H; ++r) {
            double s = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                int64_t p = (int64_t)t * k + j;
                s += w[p] * y[p * H + r];
            }
            out[(int64_t)t * H + r] = s;
        }

    if (act)
        memcpy(act, a, sizeof(double) * (size_t)(NP * I));
    free(a);
    free(y);
    return 0;
}

/* Greedy token: the first v holding the largest fp32-rounded logit. */
static int32_t first_argmax_f32(const double *z, int32_t V)
{
    int32_t best = 0;
    float best_v = (float)z[0];
    for (int32_t v = 1; v < V; ++v) {
        float zv = (float)z[v];
        if (zv > best_v) {
            best = v;
            best_v = zv;
        }
    }
    return best;
}

int oracle_lmhead(const uint16_t *h, const uint16_t *wlm,
                  int32_t M, int32_t H, int32_t V,
                  int32_t *tok, double *zmax, double *gap)
{
    if (!h || !wlm || !tok || !zmax || !gap)
        return -1;
    if (M < 1 || H < 1 || V < 1)
        return -2;
    if (!all_finite_bf16(h, (int64_t)M * H) ||
        !all_finite_bf16(wlm, (int64_t)V * H))
        return -4;

    double *z = (double *)malloc(sizeof(double) * (size_t)V);
    for (int32_t t = 0; t < M; ++t) {
        /* Logits of token t over the whole vocabulary. */
#pragma omp parallel for schedule(static)
        for (int32_t v = 0; v < V; ++v)
            z[v] = dot_bf16(h + (int64_t)t * H, wlm + (int64_t)v * H, H);

        int32_t best = first_argmax_f32(z, V);
        tok[t] = best;
        zmax[t] = z[best];

        double unused;
        sorted_gaps(z, V, 1, &gap[t], &unused);
    }
    free(z);
    return 0;
}

int oracle_greedy_verdict(const int32_t *tokens, const int32_t *tok, int32_t M,
                          int32_t *accept)
{
    if (!tokens || !tok || !accept)
        return -1;
    if (M < 1)
        return -2;
    /* Walk the chain from the first drafted candidate: position i is
     * accepted when its token is what the target predicted after position
     * i - 1; the first rejection ends the accepted prefix. */
    int32_t n = 0;
    for (int32_t i = 1; i < M; ++i) {
        if (tokens[i] != tok[i - 1])
            break;
        n = i;
    }
    accept[0] = n + 1;
    accept[1] = tok[n];
    return 0;
}

/* Nearest bf16 value to v, ties to an even significand, as a bit pattern:
 * 8 significant bits in every binade, a fixed spacing of 2^-133 below the
 * smallest normal. nearbyint rounds to nearest even in the default mode. */
static uint16_t bf16_nearest(double v)
{
    if (v == 0.0)
        return signbit(v) ? 0x8000 : 0;
    int e;
    (void)frexp(v, &e);                 /* |v| = m * 2^e, 0.5 <= m < 1 */
    int q = e - 8;                      /* spacing of the binade holding v */
    if (q < -133)
        q = -133;
    double r = ldexp(nearbyint(ldexp(v, -q)), q);
    float f = (float)r;                 /* exact: at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

int oracle_rmsnorm(const uint16_t *h, const uint16_t *gamma, double eps,
                   int32_t M, int32_t H, uint16_t *xn, double *xn_exact)
{
    if (!h || !gamma || !xn)
        return -1;
    if (M < 1 || H < 1 || !(eps >= 0.0))
        return -2;
    if (!all_finite_bf16(h, (int64_t)M * H) || !all_finite_bf16(gamma, H))
        return -4;
    for (int32_t t = 0; t < M; ++t) {
        const uint16_t *row = h + (int64_t)t * H;
        /* mean square of the row, plus eps */
        double ss = 0.0;
        for (int32_t i = 0; i < H; ++i) {
            double v = oracle_bf16_value(row[i]);
            ss += v * v;
        }
        double ms = ss / (double)H + eps;
        if (ms == 0.0)
            return -4;
        double inv = 1.0 / sqrt(ms);
        for (int32_t i = 0; i < H; ++i) {
            double y = oracle_bf16_value(row[i]) * oracle_bf16_value(gamma[i]) * inv;
            xn[(int64_t)t * H + i] = bf16_nearest(y);
            if (xn_exact)
                xn_exact[(int64_t)t * H + i] = y;
        }
    }
    return 0;
}

double oracle_e4m3_value(uint8_t q)
{
    int sign = q >> 7, e = (q >> 3) & 15, m = q & 7;
    if (e == 15 && m == 7)
        return NAN;
    double mag = e == 0 ? ldexp((double)m / 8.0, -6)          /* subnormal */
                        : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

static int all_finite_e4m3(const uint8_t *q, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if ((q[i] & 0x7F) == 0x7F)
            return 0;
    return 1;
}

/* x (bf16) . one fp8 row times its scale, in double, ascending index:
 * every element is dequantised (code value times the row's scale) first. */
static double dot_e4m3(const uint8_t *q, double scale, const uint16_t *x, int64_t n)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i)
        s += (oracle_e4m3_value(q[i]) * scale) * oracle_bf16_value(x[i]);
    return s;
}

int oracle_expert_ffn_fp8(const uint16_t *x, const int32_t *idx, const double *w,
                          const uint8_t *qgate, const float *sgate,
                          const uint8_t *qup, const float *sup,
                          const uint8_t *qdown, const float *sdown,
                          int32_t M, int32_t H, int32_t I, int32_t E, int32_t k,
                          double *out)
{
    if (!x || !idx || !w || !qgate || !sgate || !qup || !sup || !qdown || !sdown || !out)
        return -1;
    if (M < 1 || H < 1 || I < 1 || E < 1 || k < 1)
        return -2;
    const int64_t NP = (int64_t)M * k;
    for (int64_t p = 0; p < NP; ++p)
        if (idx[p] < 0 || idx[p] >= E)
            return -3;
    if (!all_finite_bf16(x, (int64_t)M * H))
        return -4;
    for (int64_t p = 0; p < NP; ++p) {
        int64_t e = idx[p];
        if (!isfinite(w[p]) ||
            !all_finite_e4m3(qgate + e * I * H, (int64_t)I * H) ||
            !all_finite_e4m3(qup + e * I * H, (int64_t)I * H) ||
            !all_finite_e4m3(qdown + e * H * I, (int64_t)H * I))
            return -4;
        for (int32_t i = 0; i < I; ++i)
            if (!isfinite(sgate[e * I + i]) || !isfinite(sup[e * I + i]))
                return -4;
        for (int32_t r = 0; r < H; ++r)
            if (!isfinite(sdown[e * H + r]))
                return -4;
    }

    double *a = (double *)malloc(sizeof(double) * (size_t)(NP * I));

    /* Up projection and SwiGLU per pair, on the dequantised rows. */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t p = 0; p < NP; ++p)
        for (int32_t i = 0; i < I; ++i) {
            int32_t t = (int32_t)(p / k);
            int64_t e = idx[p];
            const uint16_t *xt = x + (int64_t)t * H;
            double g = dot_e4m3(qgate + (e * I + i) * H, sgate[e * I + i], xt, H);
            double u = dot_e4m3(qup + (e * I + i) * H, sup[e * I + i], xt, H);
            a[p * I + i] = swiglu(g, u);
        }

    /* Down projection and the weighted combine, slots in order. */
#pragma omp parallel for collapse(2) schedule(static)
    for (int32_t t = 0; t < M; ++t)
        for (int32_t r = 0; r < H; ++r) {
            double acc = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                int64_t p = (int64_t)t * k + j;
                int64_t e = idx[p];
                const uint8_t *row = qdown + (e * H + r) * I;
                double sd = sdown[e * H + r], y = 0.0;
                for (int32_t i = 0; i < I; ++i)
                    y += (oracle_e4m3_value(row[i]) * sd) * a[p * I + i];
                acc += w[p] * y;
            }
            out[(int64_t)t * H + r] = acc;
        }
    free(a);
    return 0;
}

int oracle_lmhead_fp8(const uint16_t *h, const uint8_t *qlm, const float *slm,
                      int32_t M, int32_t H, int32_t V,
                      int32_t *tok, double *zmax, double *gap)
{
    if (!h || !qlm || !slm || !tok || !zmax || !gap)
        return -1;
    if (M < 1 || H < 1 || V < 1)
        return -2;
    if (!all_finite_bf16(h, (int64_t)M * H) || !all_finite_e4m3(qlm, (int64_t)V * H))
        return -4;
    for (int32_t v = 0; v < V; ++v)
        if (!isfinite(slm[v]))
            return -4;
    double *z = (double *)malloc(sizeof(double) * (size_t)V);
    for (int32_t t = 0; t < M; ++t) {
#pragma omp parallel for schedule(static)
        for (int32_t v = 0; v < V; ++v)
            z[v] = dot_e4m3(qlm + (int64_t)v * H, slm[v], h + (int64_t)t * H, H);
        int32_t best = first_argmax_f32(z, V);
        tok[t] = best;
        zmax[t] = z[best];
        double unused;
        sorted_gaps(z, V, 1, &gap[t], &unused);
    }
    free(z);
    return 0;
}
