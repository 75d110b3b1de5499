// route.hip -- router gate GEMV + softmax top-k (moe_route).
//
// Router chain of the LMSYS post "Chasing the batch-1 floor: Ling-3.0-flash
// speculative decode on Blackwell", section "PDL: the latency floor of
// stacked small kernels", Fig. 7: gate matvec, then top-k. The gate weight
// is bf16 (section "bf16 router gate and lm_head").
//
// The post hides the gate's 2.6 MB cold read behind its producer with a
// programmatic dependent launch. Here the chain is one launch whose latency
// is a single HBM round trip plus the selection:
//   - a group of RT router rows (8 rows with two column blocks packed per
//     v_mfma_f32_16x16x32_bf16 up to 8 tokens, else 16 rows) is split along
//     the hidden dimension over KS workgroups (4 when every wavefront would
//     otherwise take at least four steps), so the cold read is spread over
//     all CUs; each workgroup's wavefronts split its slice again. Every
//     wavefront issues all of its weight loads and hidden-state loads (the
//     latter hit in L2) at once, then runs one MFMA per 32 (or 64) columns.
//     The partial tiles are added in LDS in a fixed order and each slice's
//     partial logits published with device-scope stores;
//   - the last workgroup to arrive (two-level ticket counted with
//     agent-scope releases and acquired on the chain; no spinning) adds each
//     logit's slice partials in slice order and the bias, then selects, one
//     wavefront per token:
//     every lane sorts its logits by (value descending, id ascending) once;
//     then each of the k rounds takes the wave-wide maximum of the lane heads
//     (DPP on the 32-bit order code), breaks an equal-value tie by the
//     lowest id, and advances the winning lane's list. All loads are
//     unpredicated and every step is branch-free apart from uniform tie
//     checks. The softmax of the selected logits is taken in fp32.
//   - moe_route_rmsnorm puts the chain's norm in front (Fig. 7: norm -> gate
//     matvec -> top-k), read as RMSNorm with a per-column gain: every lane
//     already holds its chunks of the hidden states and loads the same
//     lane's chunks of the other slices, so the sum of squares is taken
//     from registers (per lane in slice and step order, then over the lanes
//     of a token in a fixed order through LDS), each lane scales its chunks
//     and rounds them once to bf16 before the MFMAs, and the workgroups of
//     row group 0 write the normalised rows for the expert kernels. Every
//     workgroup computes the same bits.
#include "common.h"
#include "select.h"

#include <utility>

namespace mv {

typedef float f32x2 __attribute__((ext_vector_type(2)));

// bf16(x * gain * inv) for eight elements: x * gain is exact in fp32 (two
// 8-bit significands), then one product and one rounding to bf16
// (v_cvt_pk_bf16_f32: nearest, ties to even, in the default mode)
__device__ __forceinline__ u32x4 rmsnorm8_bf16(u32x4 v, u32x4 g, float inv)
{
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float xl = __builtin_bit_cast(float, v[i] << 16);
        const float xh = __builtin_bit_cast(float, v[i] & 0xFFFF0000u);
        const float gl = __builtin_bit_cast(float, g[i] << 16);
        const float gh = __builtin_bit_cast(float, g[i] & 0xFFFF0000u);
        const f32x2 y = {(xl * gl) * inv, (xh * gh) * inv};
        r[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(y, bf16x2));
    }
    return r;
}

// S: MFMA steps per wavefront; KJ: logits per lane in the selection (a
// power of two, KJ * 64 >= E; 0: no arrival and no selection, the kernel
// ends once its partial logits are out); RT: router rows per workgroup; P: column
// blocks per MFMA. With P = 2 (RT = 8 rows, at most 8 tokens) one MFMA takes
// two 32-column blocks at once, block-diagonally: tile rows 0-7 and tokens
// 0-7 carry block X, tile rows 8-15 and tokens 8-15 carry block Y (the same
// router rows and tokens), so D[r][t] + D[8+r][8+t] is the dot product over
// 64 columns and every lane loads distinct data.
// W: wavefronts per workgroup; in the selecting workgroup each takes one
// token at a time. KS: workgroups per group of router rows, each taking
// 1/KS of the hidden dimension (slice q = its index mod KS; inside it the
// W wavefronts split the columns again), so that the cold read is spread
// over KS times more CUs; their partial logits plog[q][t][e] are added in
// slice order, then the bias, by the selecting workgroup.
template <int S, int KJ, int RT, int P, bool NORM, int W, int KS>
__global__ __launch_bounds__(W * kWave) void route_kernel(
    const u32x4 *__restrict__ x, const u32x4 *__restrict__ wr,
    const float *__restrict__ bias, int M, int H, int E, int k,
    float *__restrict__ plog, float *__restrict__ logits, int *__restrict__ topk_idx,
    float *__restrict__ topk_w, unsigned *__restrict__ ticket,
    const u32x4 *__restrict__ gamma, float eps, u32x4 *__restrict__ xn_out)
{
    static_assert(RT == 8 || RT == 16, "tile rows");
    static_assert(P == 1 || (P == 2 && RT == 8), "block-diagonal packing needs 8-row tiles");
    static_assert(!NORM || S <= 16, "the norm needs every hidden-state chunk in registers at once");
    __shared__ f32x4 s_part[W][kWave];
    __shared__ float s_ss[NORM ? W : 1][kWave];
    __shared__ int s_last;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nch = H / 8;                       // 16-byte chunks per row
    const int j = lane & 15;                     // A row in the tile / B column
    const int g = lane >> 4;                     // chunk within a 32-column block
    const int blk = P == 2 ? j >> 3 : 0;         // column block of this lane
    const int ks = KS > 1 ? (int)(blockIdx.x % KS) : 0;   // this workgroup's slice
    const int e0 = (int)(blockIdx.x / KS) * RT;

    // ---- every load first, unpredicated: rows past E, tokens past M and
    // chunks past the row end read valid memory (zeroed or unused below)
    int arow = e0 + (P == 2 ? (j & 7) : (j % RT));
    arow = arow < E ? arow : E - 1;
    int tok = P == 2 ? (j & 7) : j;
    tok = tok < M ? tok : M - 1;
    const u32x4 *ap = wr + (size_t)arow * nch;
    const u32x4 *bp = x + (size_t)tok * nch;
    // first chunk of this lane in slice q (then every 4P chunks, S steps)
    auto chunk0 = [&](int q) { return (q * W + wave) * (4 * P * S) + 4 * blk + g; };
    const int cbase = chunk0(ks);
    // at most 16 steps of operands in registers at a time
    constexpr int SPH = S < 16 ? S : 16;
    static_assert(S % SPH == 0, "steps per phase");
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    u32x4 xn_keep[NORM ? SPH : 1];               // the normalised chunks, stored late
#pragma unroll
    for (int ph = 0; ph < S; ph += SPH) {
        u32x4 a[SPH], b[SPH], gm[NORM ? SPH : 1];
#pragma unroll
        for (int s = 0; s < SPH; ++s) {
            const int c = cbase + 4 * P * (ph + s);
            a[s] = load_stream(ap + (c < nch ? c : nch - 1));
        }
#pragma unroll
        for (int s = 0; s < SPH; ++s) {
            const int c = cbase + 4 * P * (ph + s);
            b[s] = bp[c < nch ? c : nch - 1];
            if constexpr (NORM)
                gm[s] = gamma[c < nch ? c : nch - 1];
        }
        // with the norm, the same lane's chunks of the other slices too
        // (slices in order, this workgroup's own left out): the squares
        // cover the whole row in every workgroup
        u32x4 xo[NORM && KS > 1 ? KS - 1 : 1][NORM ? SPH : 1];
        if constexpr (NORM && KS > 1) {
#pragma unroll
            for (int q = 0; q < KS - 1; ++q) {
                const int qa = q < ks ? q : q + 1;
#pragma unroll
                for (int s = 0; s < SPH; ++s) {
                    const int c = chunk0(qa) + 4 * P * s;
                    xo[q][s] = bp[c < nch ? c : nch - 1];
                }
            }
        }
        wait_vmcnt<0>();
        if constexpr (NORM) {
            // this lane's squares, slices in order, steps in order; then, in
            // every wavefront, each lane adds the W wavefronts' values of its
            // own lane slot, and an xor butterfly over the lanes that hold
            // the same token (j = t and, packed, t + 8; every g) completes
            // the row: one fixed order, the same in every lane and workgroup
            float ss = 0.0f;
#pragma unroll
            for (int qa = 0; qa < KS; ++qa) {
#pragma unroll
                for (int s = 0; s < SPH; ++s) {
                    u32x4 v = b[s];
                    if constexpr (KS > 1) {
                        // slice qa is xo[qa] below this workgroup's, xo[qa - 1] above
                        const u32x4 lo = xo[qa < KS - 1 ? qa : KS - 2][s];
                        const u32x4 hi = xo[qa > 0 ? qa - 1 : 0][s];
                        v = qa < ks ? lo : (qa > ks ? hi : v);
                    }
                    const float q = dot8_bf16(v, v, 0.0f);     // v_dot2_f32_bf16
                    ss += chunk0(qa) + 4 * P * s < nch ? q : 0.0f;
                }
            }
            s_ss[wave][lane] = ss;
            __syncthreads();
            float tot = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w)
                tot += s_ss[w][lane];
            if (P == 2)
                tot += __shfl_xor(tot, 8);
            tot += __shfl_xor(tot, 16);
            tot += __shfl_xor(tot, 32);
            const float inv = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
            for (int s = 0; s < SPH; ++s) {
                b[s] = rmsnorm8_bf16(b[s], gm[s], inv);
                xn_keep[s] = b[s];
            }
        }
        // partial tile over this wavefront's columns
#pragma unroll
        for (int s = 0; s < SPH; ++s) {
            const bool ok = cbase + 4 * P * (ph + s) < nch;
            acc = mfma_bf16(ok ? a[s] : u32x4{0, 0, 0, 0}, ok ? b[s] : u32x4{0, 0, 0, 0}, acc);
        }
    }
    s_part[wave][lane] = acc;
    __syncthreads();

    // ---- the partial tiles in a fixed order; lane (j, g) holds rows
    // 4g .. 4g+3 of the tile for column j (with P = 2 the Y block of the
    // same rows and token sits 40 lanes up)
    if (wave == 0) {
        f32x4 sum = s_part[0][lane];
#pragma unroll
        for (int w = 1; w < W; ++w)
            sum += s_part[w][lane];
        if (P == 2) {
            const int ly = (lane + 40) & (kWave - 1);
            f32x4 sy = s_part[0][ly];
#pragma unroll
            for (int w = 1; w < W; ++w)
                sy += s_part[w][ly];
            sum += sy;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * g + r, e = e0 + row;
            if (row < RT && e < E && j < M && (P == 1 || j < 8))
                __hip_atomic_store(plog + ((size_t)ks * M + j) * E + e, sum[r],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // ---- KJ = 0: the partial logits are the result (moe_layer: the up
    // projection's prologue selects); with the norm, row group 0's
    // workgroups also write the normalised rows
    if constexpr (KJ == 0) {
        if constexpr (NORM) {
            if (e0 == 0 && (P == 2 ? (j & 7) : j) < M) {
#pragma unroll
                for (int s = 0; s < SPH; ++s) {
                    const int c = cbase + 4 * P * s;
                    if (c < nch)
                        xn_out[(size_t)tok * nch + c] = xn_keep[s];
                }
            }
        }
        return;
    } else {
        // ---- the last workgroup to arrive selects. Wave 0 stored this
        // workgroup's partial logits; thread 0 (of wave 0) releases them with its
        // arrival and the last arrival acquires them (two-level arrival)
        __syncthreads();
        if (threadIdx.x == 0)
            s_last = arrive_last(ticket);
        __syncthreads();
        if constexpr (NORM) {
            // the workgroups of row group 0 (one per slice) write the
            // normalised rows for the expert kernels only now: they must land by
            // the end of the kernel, not before the ticket, so their latency
            // overlaps the selection
            if (e0 == 0 && (P == 2 ? (j & 7) : j) < M) {
#pragma unroll
                for (int s = 0; s < SPH; ++s) {
                    const int c = cbase + 4 * P * s;
                    if (c < nch)
                        xn_out[(size_t)tok * nch + c] = xn_keep[s];
                }
            }
        }
        if (!s_last)
            return;
        if (threadIdx.x == 0)
            __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

        for (int t = wave; t < M; t += W) {
            // this lane's logits e = lane + 64*q as (order code, id); ids past E
            // get code 0, below every number (k <= E keeps them unselected)
            float lv[KJ], pv[KS][KJ], bq[KJ];
#pragma unroll
            for (int q = 0; q < KJ; ++q) {           // all loads in flight together
                const int e = lane + kWave * q, ec = e < E ? e : E - 1;
#pragma unroll
                for (int sl = 0; sl < KS; ++sl)
                    pv[sl][q] = __hip_atomic_load(plog + ((size_t)sl * M + t) * E + ec,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                bq[q] = bias ? bias[ec] : 0.0f;
            }
#pragma unroll
            for (int q = 0; q < KJ; ++q) {
                const int e = lane + kWave * q;
                // the slices' partial sums in slice order, then the bias
                float l = pv[0][q];
#pragma unroll
                for (int sl = 1; sl < KS; ++sl)
                    l += pv[sl][q];
                lv[q] = l + bq[q];
                if (logits && e < E)
                    logits[(size_t)t * E + e] = lv[q];
            }
            int sel_i;
            float sel_w;
            topk_select<KJ>(lv, E, k, lane, sel_i, sel_w);
            if (lane < k) {
                topk_idx[(size_t)t * k + lane] = sel_i;
                topk_w[(size_t)t * k + lane] = sel_w;
            }
        }
    }
}

// the optional norm: gain [H] bf16, eps, normalised rows out [M,H] bf16
struct RouteNorm {
    const uint16_t *gamma;
    float eps;
    uint16_t *xn;
    int *ks_out;                 // the launch's number of slices of the hidden dimension
};

// RT router rows per workgroup, W wavefronts, KS workgroups per row group
template <int S, int KJ, int RT, int P, int W, int KS>
static moe_status_t launch_route4(const uint16_t *x, const uint16_t *w, const float *bias,
                                  int M, int H, int E, int k, float *plog, float *logits,
                                  int *idx, float *tw, unsigned *ticket, const RouteNorm &nm,
                                  hipStream_t st)
{
    nm.ks_out[0] = KS;
    const int grid = (E + RT - 1) / RT * KS;
    if ((grid + kArrivalGroup - 1) / kArrivalGroup > kWsGroups)
        return MOE_ERR_UNSUPPORTED;                      // (E <= 1024 stays within)
    if (nm.gamma) {
        if constexpr (S <= 128 / W)
            hipLaunchKernelGGL((route_kernel<S, KJ, RT, P, true, W, KS>), dim3(grid),
                               dim3(W * kWave), 0, st, (const u32x4 *)x, (const u32x4 *)w, bias,
                               M, H, E, k, plog, logits, idx, tw, ticket,
                               (const u32x4 *)nm.gamma, nm.eps, (u32x4 *)nm.xn);
        else
            return MOE_ERR_UNSUPPORTED;
    } else {
        hipLaunchKernelGGL((route_kernel<S, KJ, RT, P, false, W, KS>), dim3(grid),
                           dim3(W * kWave), 0, st, (const u32x4 *)x, (const u32x4 *)w, bias, M,
                           H, E, k, plog, logits, idx, tw, ticket, nullptr, 0.0f, nullptr);
    }
    return check_launch();
}

// Rows whose columns take at least four steps of every wavefront are
// split over kRouteSlices workgroups when the grid stays within two
// workgroups per CU: the 2.6 MB gate of 512 x 2560 then streams through
// 256 CUs instead of 64.
constexpr int kRouteSlices = kRouteSlicesMax;
template <int S, int KJ, int RT, int P, int W>
static moe_status_t launch_route3(const uint16_t *x, const uint16_t *w, const float *bias,
                                  int M, int H, int E, int k, float *plog, float *logits,
                                  int *idx, float *tw, unsigned *ticket, const RouteNorm &nm,
                                  hipStream_t st)
{
    if constexpr (S >= kRouteSlices) {
        if ((E + RT - 1) / RT * kRouteSlices <= 2 * 256)   // (at most 16 arrival groups)
            return launch_route4<(S + kRouteSlices - 1) / kRouteSlices, KJ, RT, P, W,
                                 kRouteSlices>(x, w, bias, M, H, E, k, plog, logits, idx, tw,
                                               ticket, nm, st);
    }
    return launch_route4<S, KJ, RT, P, W, 1>(x, w, bias, M, H, E, k, plog, logits, idx, tw,
                                             ticket, nm, st);
}

// S counts the 32-column MFMA steps of eight wavefronts. Up to 8 tokens:
// 8-row tiles, two blocks packed per step, eight wavefronts. More tokens
// fill a 16-row tile with 16 distinct rows and 16 token columns; sixteen
// wavefronts (up to 512 experts) then halve the steps of each and select
// one token each.
template <int S, int KJ>
static moe_status_t launch_route2(const uint16_t *x, const uint16_t *w, const float *bias,
                                  int M, int H, int E, int k, float *plog, float *logits,
                                  int *idx, float *tw, unsigned *ticket, const RouteNorm &nm,
                                  hipStream_t st)
{
    // (the selection's keys and partial sums of more than 512 experts need
    // the register budget of eight wavefronts)
    constexpr int W = KJ <= 8 ? 16 : 8;
    if (M <= 8)
        return launch_route3<(S + 1) / 2, KJ, 8, 2, 8>(x, w, bias, M, H, E, k, plog, logits,
                                                       idx, tw, ticket, nm, st);
    return launch_route3<(S * 8 + W - 1) / W, KJ, 16, 1, W>(x, w, bias, M, H, E, k, plog,
                                                            logits, idx, tw, ticket, nm, st);
}

template <int S>
static moe_status_t launch_route(const uint16_t *x, const uint16_t *w, const float *bias,
                                 int M, int H, int E, int k, float *plog, float *logits,
                                 int *idx, float *tw, unsigned *ticket, const RouteNorm &nm,
                                 bool select, hipStream_t st)
{
    if (!select)                 // partial logits only
        return launch_route2<S, 0>(x, w, bias, M, H, E, k, plog, logits, idx, tw, ticket, nm, st);
    if (E <= 128)
        return launch_route2<S, 2>(x, w, bias, M, H, E, k, plog, logits, idx, tw, ticket, nm, st);
    if (E <= 256)
        return launch_route2<S, 4>(x, w, bias, M, H, E, k, plog, logits, idx, tw, ticket, nm, st);
    if (E <= 512)
        return launch_route2<S, 8>(x, w, bias, M, H, E, k, plog, logits, idx, tw, ticket, nm, st);
    return launch_route2<S, 16>(x, w, bias, M, H, E, k, plog, logits, idx, tw, ticket, nm, st);
}

// Workspace: the header (ticket), then the partial logits [KS][M][E] fp32
// of up to kRouteSlices slices.
static size_t route_ws_logits(int32_t M, int32_t E)
{
    return align_up((size_t)kRouteSlices * M * (size_t)E * sizeof(float), 256);
}

// 32-column MFMA steps of each of eight wavefronts
static int route_need(int H)
{
    return (H / 8 + 4 * 8 - 1) / (4 * 8);
}

// the norm needs every chunk of a lane in registers at once: at most 16
// MFMA steps per lane with eight wavefronts (M <= 8, any H up to 8192), at
// most 8 with sixteen, whose register budget is half (H <= 4096)
bool route_norm_supported(int32_t M, int32_t H)
{
    return (route_need(H) + 1) / 2 <= (M <= 8 ? 16 : 8);
}

// select = false: the kernel stops at the partial logits (plog in the
// workspace, *ks slices of the hidden dimension), which the caller's next
// kernel selects from.
moe_status_t route_enqueue(const uint16_t *x, const uint16_t *w_router,
                           const float *bias, int32_t M, int32_t H, int32_t E,
                           int32_t k, int32_t *topk_idx, float *topk_w,
                           float *logits, void *ws, hipStream_t st,
                           const uint16_t *gamma, float eps, uint16_t *x_norm,
                           bool select, int *ks)
{
    unsigned *ticket = (unsigned *)ws;
    float *plog = (float *)((char *)ws + kWsHeader);
    int ks_local = 1;
    const RouteNorm nm{gamma, eps, x_norm, ks ? ks : &ks_local};
    const int need = route_need(H);
#define MV_ROUTE(S) launch_route<S>(x, w_router, bias, M, H, E, k, plog, logits, topk_idx, \
                                    topk_w, ticket, nm, select, st)
    if (need <= 2)
        return MV_ROUTE(2);
    if (need <= 4)
        return MV_ROUTE(4);
    if (need <= 10)
        return MV_ROUTE(10);
    if (need <= 16)
        return MV_ROUTE(16);
    return MV_ROUTE(32);
#undef MV_ROUTE
}

moe_status_t norm_check(const uint16_t *gamma, float eps, const uint16_t *x_norm,
                        int32_t M, int32_t H)
{
    if (!gamma || !x_norm)
        return MOE_ERR_NULL;
    if (!(eps >= 0.0f) || eps == INFINITY)
        return MOE_ERR_SHAPE;
    if (!aligned16(gamma) || !aligned16(x_norm))
        return MOE_ERR_ALIGN;
    if (!route_norm_supported(M, H))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status_t route_check(const uint16_t *x, const uint16_t *w_router,
                         const float *bias, int32_t M, int32_t H, int32_t E,
                         int32_t k, const int32_t *topk_idx, const float *topk_w,
                         const float *logits)
{
    if (!x || !w_router || !topk_idx || !topk_w)
        return MOE_ERR_NULL;
    moe_status_t s = check_moe_shape(M, H, E, k);
    if (s != MOE_OK)
        return s;
    if (!aligned16(x) || !aligned16(w_router) || !aligned4(topk_idx) ||
        !aligned4(topk_w) || (bias && !aligned4(bias)) ||
        (logits && !aligned4(logits)))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

} // namespace mv

using namespace mv;

extern "C" size_t moe_route_workspace_bytes(int32_t M, int32_t E)
{
    if (M < 1 || E < 1 || M > kMaxM || E > kMaxE)
        return 0;
    return kWsHeader + route_ws_logits(M, E);
}

extern "C" moe_status_t moe_route(const uint16_t *x, const uint16_t *w_router,
                                  const float *bias, int32_t M, int32_t H,
                                  int32_t E, int32_t k, int32_t *topk_idx,
                                  float *topk_w, float *logits, void *workspace,
                                  size_t workspace_bytes, void *stream)
{
    moe_status_t s = route_check(x, w_router, bias, M, H, E, k, topk_idx, topk_w, logits);
    if (s != MOE_OK)
        return s;
    if (!workspace)
        return MOE_ERR_NULL;
    if (!aligned16(workspace))
        return MOE_ERR_ALIGN;
    if (workspace_bytes < moe_route_workspace_bytes(M, E))
        return MOE_ERR_WORKSPACE;
    return route_enqueue(x, w_router, bias, M, H, E, k, topk_idx, topk_w, logits,
                         workspace, (hipStream_t)stream, nullptr, 0.0f, nullptr, true, nullptr);
}

extern "C" moe_status_t moe_route_rmsnorm(const uint16_t *h, const uint16_t *gamma,
                                          float eps, const uint16_t *w_router,
                                          const float *bias, int32_t M, int32_t H,
                                          int32_t E, int32_t k, uint16_t *x_norm,
                                          int32_t *topk_idx, float *topk_w, float *logits,
                                          void *workspace, size_t workspace_bytes,
                                          void *stream)
{
    moe_status_t s = route_check(h, w_router, bias, M, H, E, k, topk_idx, topk_w, logits);
    if (s != MOE_OK)
        return s;
    s = norm_check(gamma, eps, x_norm, M, H);
    if (s != MOE_OK)
        return s;
    if (!workspace)
        return MOE_ERR_NULL;
    if (!aligned16(workspace))
        return MOE_ERR_ALIGN;
    if (workspace_bytes < moe_route_workspace_bytes(M, E))
        return MOE_ERR_WORKSPACE;
    return route_enqueue(h, w_router, bias, M, H, E, k, topk_idx, topk_w, logits,
                         workspace, (hipStream_t)stream, gamma, eps, x_norm, true, nullptr);
}
