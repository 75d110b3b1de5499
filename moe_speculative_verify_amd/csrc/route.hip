// route.hip -- router gate GEMV + softmax top-k (moe_route).
//
// Router chain of the LMSYS post "Chasing the batch-1 floor: Ling-3.0-flash
// speculative decode on Blackwell", section "PDL: the latency floor of
// stacked small kernels", Fig. 7: gate matvec, then top-k. The gate weight
// is bf16 (section "bf16 router gate and lm_head").
//
// One launch does both steps. Every wavefront owns router rows: it issues
// its row's 128-bit weight loads first, then reads the (cached) token rows
// and reduces one fp32 dot product per token. The last workgroup to finish
// (an atomic ticket, no spinning) runs the top-k: one wavefront per token,
// k rounds of a wave-wide argmax with lower-id tie-break, then the softmax
// of the selected logits.
#include "common.h"

namespace mv {

constexpr int kRouteThreads = 128;   // two wavefronts per workgroup

template <int NC>  // NC = 16-byte chunks per lane per row (H <= 512 * NC)
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const u32x4 *__restrict__ x, const u32x4 *__restrict__ wr,
    const float *__restrict__ bias, int M, int H, int E, int k,
    float *__restrict__ logits, int *__restrict__ topk_idx,
    float *__restrict__ topk_w, unsigned *__restrict__ ticket)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwave = blockDim.x / kWave;
    const int nchunk = H / 8;

    // ---- gate GEMV: l[t,e] = x[t,:] . wr[e,:] + bias[e]
    for (int e = blockIdx.x * nwave + wave; e < E; e += gridDim.x * nwave) {
        u32x4 w[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int i = lane + kWave * c;
            w[c] = (i < nchunk) ? load_stream(wr + (size_t)e * nchunk + i)
                                : u32x4{0, 0, 0, 0};
        }
        const float b = bias ? bias[e] : 0.0f;
        for (int t = 0; t < M; ++t) {
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int i = lane + kWave * c;
                if (i < nchunk)
                    acc = dot8_bf16(w[c], x[(size_t)t * nchunk + i], acc);
            }
            acc = wave_sum(acc);
            if (lane == 0)
                logits[(size_t)t * E + e] = acc + b;
        }
    }

    // ---- the last workgroup to arrive selects
    __shared__ int s_last;
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();                         // publish this block's logits
        const unsigned prev = atomicAdd(ticket, 1u);
        s_last = (prev == gridDim.x - 1);
    }
    __syncthreads();
    if (!s_last)
        return;
    __threadfence();                             // see every block's logits
    if (threadIdx.x == 0)
        *ticket = 0u;                            // ready for the next call

    constexpr int kJ = kMaxE / kWave;            // logits held per lane

    for (int t = wave; t < M; t += nwave) {
        float v[kJ];
        uint32_t taken = 0;
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            const int e = lane + kWave * j;
            float l = -INFINITY;
            if (e < E) {
                l = logits[(size_t)t * E + e];
                if (l != l)
                    l = -INFINITY;               // NaN never outranks a number
            } else {
                taken |= 1u << j;
            }
            v[j] = l;
        }
        // lane s keeps the s-th selection
        int my_e = 0;
        float my_v = -INFINITY;
        for (int s = 0; s < k; ++s) {
            // this lane's best untaken logit; j ascending = id ascending,
            // so a strict comparison keeps the lower id on ties
            float bv = -INFINITY;
            int be = 0x7FFFFFFF;
#pragma unroll
            for (int j = 0; j < kJ; ++j) {
                const int e = lane + kWave * j;
                const bool free = !((taken >> j) & 1u);
                if (free && (v[j] > bv || (v[j] == bv && e < be))) {
                    bv = v[j];
                    be = e;
                }
            }
            // wave-wide argmax, lower id on ties
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) {
                const float ov = __shfl_xor(bv, m);
                const int oe = __shfl_xor(be, m);
                if (ov > bv || (ov == bv && oe < be)) {
                    bv = ov;
                    be = oe;
                }
            }
            if ((be & (kWave - 1)) == lane)
                taken |= 1u << (be / kWave);
            if (lane == s) {
                my_e = be;
                my_v = bv;
            }
        }
        // softmax over the selected logits, shifted by the largest
        const float top = __shfl(my_v, 0);
        const float ex = (lane < k) ? expf(my_v - top) : 0.0f;
        const float den = wave_sum(ex);
        if (lane < k) {
            topk_idx[(size_t)t * k + lane] = my_e;
            topk_w[(size_t)t * k + lane] = ex / den;
        }
    }
}

template <int NC>
static void launch_route(const uint16_t *x, const uint16_t *w, const float *bias,
                         int M, int H, int E, int k, float *logits, int *idx,
                         float *tw, unsigned *ticket, hipStream_t st)
{
    const int nwave = kRouteThreads / kWave;
    const int grid = (E + nwave - 1) / nwave;
    hipLaunchKernelGGL(route_kernel<NC>, dim3(grid), dim3(kRouteThreads), 0, st,
                       (const u32x4 *)x, (const u32x4 *)w, bias, M, H, E, k,
                       logits, idx, tw, ticket);
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
    else if (need <= 4)
        launch_route<4>(x, w_router, bias, M, H, E, k, lg, topk_idx, topk_w, ticket, st);
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
