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
//   - every wavefront owns one router row: it issues the row's 128-bit
//     loads (1 KB contiguous per instruction) before anything else, then
//     reduces one fp32 dot product per token with DPP (no LDS traffic);
//   - the logits are published with device-scope stores, and the last
//     workgroup to take a ticket (device-scope atomic; no spinning, no cache
//     flush) selects: one wavefront per token, k rounds of a wave-wide
//     (value, id) argmax with the lower id winning ties, then the softmax of
//     the selected logits in fp32.
#include "common.h"

namespace mv {

constexpr int kRouteWaves = 8;

// lexicographic (larger value, then smaller id) maximum with a DPP partner
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float &v, int &i)
{
    const float ov = dpp_f32<CTRL>(v);
    const int oi = dpp_i32<CTRL>(i);
    const bool take = ov > v || (ov == v && oi < i);
    v = take ? ov : v;
    i = take ? oi : i;
}

template <int NC, int KJ>  // NC: 16-byte chunks per lane per row; KJ: logits per lane
__global__ __launch_bounds__(kRouteWaves * kWave) void route_kernel(
    const u32x4 *__restrict__ x, const u32x4 *__restrict__ wr,
    const float *__restrict__ bias, int M, int H, int E, int k,
    float *__restrict__ logits, int *__restrict__ topk_idx,
    float *__restrict__ topk_w, unsigned *__restrict__ ticket)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nch = H / 8;

    // ---- gate GEMV: l[t,e] = x[t,:] . wr[e,:] + bias[e]
    for (int e = blockIdx.x * kRouteWaves + wave; e < E; e += gridDim.x * kRouteWaves) {
        u32x4 w[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int ci = lane + kWave * c;
            w[c] = (ci < nch) ? load_stream(wr + (size_t)e * nch + ci) : u32x4{0, 0, 0, 0};
        }
        const float b = bias ? bias[e] : 0.0f;
        for (int t = 0; t < M; ++t) {
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int ci = lane + kWave * c;
                if (ci < nch)
                    acc = dot8_bf16(w[c], x[(size_t)t * nch + ci], acc);
            }
            acc = wave_sum(acc);
            if (lane == 0)
                __hip_atomic_store(logits + (size_t)t * E + e, acc + b, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // ---- the last workgroup to arrive selects
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);               // this thread's logits are out
    __syncthreads();
    if (threadIdx.x == 0)
        s_last = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
    __syncthreads();
    if (!s_last)
        return;
    if (threadIdx.x == 0)
        __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    for (int t = wave; t < M; t += kRouteWaves) {
        float v[KJ];
        uint32_t taken = 0;
#pragma unroll
        for (int jj = 0; jj < KJ; ++jj) {
            const int e = lane + kWave * jj;
            float l = -INFINITY;
            if (e < E) {
                l = __hip_atomic_load(logits + (size_t)t * E + e, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
                if (l != l)
                    l = -INFINITY;               // NaN never outranks a number
            } else {
                taken |= 1u << jj;
            }
            v[jj] = l;
        }
        int my_e = 0;                            // lane s keeps selection s
        float my_v = -INFINITY;
        for (int s = 0; s < k; ++s) {
            // this lane's best free logit; jj ascending = id ascending
            float bv = -INFINITY;
            int be = 0x7FFFFFFF;
#pragma unroll
            for (int jj = 0; jj < KJ; ++jj) {
                const int e = lane + kWave * jj;
                if (!((taken >> jj) & 1u) && (v[jj] > bv || (v[jj] == bv && e < be))) {
                    bv = v[jj];
                    be = e;
                }
            }
            argmax_dpp<kDppXor1>(bv, be);
            argmax_dpp<kDppXor2>(bv, be);
            argmax_dpp<kDppHalfMirror>(bv, be);
            argmax_dpp<kDppMirror>(bv, be);
            // the four row winners, in a fixed order
            float wv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), 0));
            int wi = __builtin_amdgcn_readlane(be, 0);
#pragma unroll
            for (int r = 1; r < 4; ++r) {
                const float cv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), 16 * r));
                const int ci = __builtin_amdgcn_readlane(be, 16 * r);
                if (cv > wv || (cv == wv && ci < wi)) {
                    wv = cv;
                    wi = ci;
                }
            }
            if ((wi & (kWave - 1)) == lane)
                taken |= 1u << (wi / kWave);
            if (lane == s) {
                my_e = wi;
                my_v = wv;
            }
        }
        // softmax over the selected logits, shifted by the largest
        const float top = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_v), 0));
        const float ex = (lane < k) ? expf(my_v - top) : 0.0f;
        const float den = wave_sum(ex);
        if (lane < k) {
            topk_idx[(size_t)t * k + lane] = my_e;
            topk_w[(size_t)t * k + lane] = ex / den;
        }
    }
}

template <int NC, int KJ>
static void launch_route2(const uint16_t *x, const uint16_t *w, const float *bias,
                          int M, int H, int E, int k, float *logits, int *idx,
                          float *tw, unsigned *ticket, hipStream_t st)
{
    const int grid = (E + kRouteWaves - 1) / kRouteWaves;
    hipLaunchKernelGGL((route_kernel<NC, KJ>), dim3(grid), dim3(kRouteWaves * kWave), 0,
                       st, (const u32x4 *)x, (const u32x4 *)w, bias, M, H, E, k,
                       logits, idx, tw, ticket);
}

template <int NC>
static void launch_route(const uint16_t *x, const uint16_t *w, const float *bias,
                         int M, int H, int E, int k, float *logits, int *idx,
                         float *tw, unsigned *ticket, hipStream_t st)
{
    if (E <= 64)
        launch_route2<NC, 1>(x, w, bias, M, H, E, k, logits, idx, tw, ticket, st);
    else if (E <= 128)
        launch_route2<NC, 2>(x, w, bias, M, H, E, k, logits, idx, tw, ticket, st);
    else if (E <= 256)
        launch_route2<NC, 4>(x, w, bias, M, H, E, k, logits, idx, tw, ticket, st);
    else if (E <= 512)
        launch_route2<NC, 8>(x, w, bias, M, H, E, k, logits, idx, tw, ticket, st);
    else
        launch_route2<NC, 16>(x, w, bias, M, H, E, k, logits, idx, tw, ticket, st);
}

// Workspace: the header (ticket), then [M,E] fp32 logits scratch.
static size_t route_ws_logits(int32_t M, int32_t E)
{
    return align_up((size_t)M * (size_t)E * sizeof(float), 256);
}

moe_status_t route_enqueue(const uint16_t *x, const uint16_t *w_router,
                           const float *bias, int32_t M, int32_t H, int32_t E,
                           int32_t k, int32_t *topk_idx, float *topk_w,
                           float *logits, void *ws, hipStream_t st)
{
    unsigned *ticket = (unsigned *)ws;
    float *lg = logits ? logits : (float *)((char *)ws + kWsHeader);
    const int need = (H / 8 + kWave - 1) / kWave;
    if (need <= 1)
        launch_route<1>(x, w_router, bias, M, H, E, k, lg, topk_idx, topk_w, ticket, st);
    else if (need <= 2)
        launch_route<2>(x, w_router, bias, M, H, E, k, lg, topk_idx, topk_w, ticket, st);
    else if (need <= 5)
        launch_route<5>(x, w_router, bias, M, H, E, k, lg, topk_idx, topk_w, ticket, st);
    else if (need <= 8)
        launch_route<8>(x, w_router, bias, M, H, E, k, lg, topk_idx, topk_w, ticket, st);
    else
        launch_route<16>(x, w_router, bias, M, H, E, k, lg, topk_idx, topk_w, ticket, st);
    return check_launch();
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
                         workspace, (hipStream_t)stream);
}
