// lmhead.hip -- lm_head GEMV fused with the greedy argmax (lmhead_argmax).
//
// The LMSYS post "Chasing the batch-1 floor: Ling-3.0-flash speculative
// decode on Blackwell" runs the lm_head in bf16 because at batch 1 it is a
// pure weight read (section "bf16 router gate and lm_head"); its logits feed
// the greedy verdict inside the verify step (section "The shape of a
// single-request step", Fig. 3).
//
// Workgroup b owns a contiguous slice of vocabulary rows; each wavefront
// streams RB rows at a time with 128-bit loads, reduces one fp32 dot per
// token and row, and keeps a running (max, first index) per token. The
// workgroup's best per token goes to a slot of the workspace; the last
// workgroup to finish (atomic ticket, no spinning) reduces the slots in
// ascending workgroup order. Logits never reach memory, and the result is
// the same whatever the finishing order.
#include "common.h"

namespace mv {

constexpr int kLmThreads = 256;
constexpr int kLmMaxGrid = 2048;

template <int NC, int RB, int MT>  // MT >= M: tokens held in registers
__global__ __launch_bounds__(kLmThreads) void lmhead_kernel(
    const u32x4 *__restrict__ h, const u32x4 *__restrict__ wl, int M, int H,
    int V, int rows_per_wg, float *__restrict__ part_v, int *__restrict__ part_i,
    unsigned *__restrict__ ticket, int *__restrict__ argmax,
    float *__restrict__ max_logit)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwave = blockDim.x / kWave;
    const int nchunk = H / 8;

    const int v0 = blockIdx.x * rows_per_wg;
    const int v1 = min(V, v0 + rows_per_wg);
    const int per_w = ((v1 - v0 + nwave - 1) / nwave + RB - 1) / RB * RB;
    const int a0 = v0 + wave * per_w;
    const int a1 = min(v1, a0 + per_w);

    float bv[MT];
    int bi[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        bv[t] = -INFINITY;
        bi[t] = 0x7FFFFFFF;
    }

    for (int v = a0; v < a1; v += RB) {
        u32x4 W[RB][NC];
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int ci = lane + kWave * c;
                W[b][c] = (v + b < a1 && ci < nchunk)
                              ? load_stream(wl + (size_t)(v + b) * nchunk + ci)
                              : u32x4{0, 0, 0, 0};
            }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t < M) {
                u32x4 xv[NC];
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int ci = lane + kWave * c;
                    xv[c] = (ci < nchunk) ? h[(size_t)t * nchunk + ci] : u32x4{0, 0, 0, 0};
                }
#pragma unroll
                for (int b = 0; b < RB; ++b) {
                    float acc = 0.0f;
#pragma unroll
                    for (int c = 0; c < NC; ++c)
                        acc = dot8_bf16(W[b][c], xv[c], acc);
                    acc = wave_sum(acc);
                    // rows ascend, so a strict comparison keeps the first
                    if (v + b < a1 && acc > bv[t]) {
                        bv[t] = acc;
                        bi[t] = v + b;
                    }
                }
            }
        }
    }

    // workgroup best per token: wavefronts in ascending row order
    __shared__ float s_v[kLmThreads / kWave][MT];
    __shared__ int s_i[kLmThreads / kWave][MT];
    if (lane == 0)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            s_v[wave][t] = bv[t];
            s_i[wave][t] = bi[t];
        }
    __syncthreads();
    if (threadIdx.x < M) {
        const int t = threadIdx.x;
        float best = s_v[0][t];
        int besti = s_i[0][t];
        for (int w = 1; w < nwave; ++w)
            if (s_v[w][t] > best || (s_v[w][t] == best && s_i[w][t] < besti)) {
                best = s_v[w][t];
                besti = s_i[w][t];
            }
        part_v[(size_t)blockIdx.x * M + t] = best;
        part_i[(size_t)blockIdx.x * M + t] = besti;
    }

    __shared__ int s_last;
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const unsigned prev = atomicAdd(ticket, 1u);
        s_last = (prev == gridDim.x - 1);
    }
    __syncthreads();
    if (!s_last)
        return;
    __threadfence();
    if (threadIdx.x == 0)
        *ticket = 0u;

    // one wavefront per token over all workgroup slots
    for (int t = wave; t < M; t += nwave) {
        float best = -INFINITY;
        int besti = 0x7FFFFFFF;
        for (int b = lane; b < (int)gridDim.x; b += kWave) {
            const float pv = part_v[(size_t)b * M + t];
            const int pi = part_i[(size_t)b * M + t];
            if (pv > best || (pv == best && pi < besti)) {
                best = pv;
                besti = pi;
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            const float ov = __shfl_xor(best, m);
            const int oi = __shfl_xor(besti, m);
            if (ov > best || (ov == best && oi < besti)) {
                best = ov;
                besti = oi;
            }
        }
        if (lane == 0) {
            argmax[t] = besti;
            if (max_logit)
                max_logit[t] = best;
        }
    }
}

static int lm_grid(int V) { return V < kLmMaxGrid ? V : kLmMaxGrid; }

template <int NC, int MT>
static void launch_lm(const uint16_t *h, const uint16_t *w, int M, int H, int V,
                      float *pv, int *pi, unsigned *ticket, int *am, float *ml,
                      hipStream_t st)
{
    // 512 workgroups cover the 256 CUs twice; small vocabularies get fewer
    int grid = (V + 63) / 64;
    if (grid > 512)
        grid = 512;
    const int rows = (V + grid - 1) / grid;
    grid = (V + rows - 1) / rows;
    // rows in flight per wavefront: fewer for wide rows to stay in registers
    constexpr int RB = NC <= 5 ? 4 : (NC <= 8 ? 2 : 1);
    hipLaunchKernelGGL((lmhead_kernel<NC, RB, MT>), dim3(grid), dim3(kLmThreads), 0,
                       st, (const u32x4 *)h, (const u32x4 *)w, M, H, V, rows, pv,
                       pi, ticket, am, ml);
}

template <int NC>
static void launch_lm_m(const uint16_t *h, const uint16_t *w, int M, int H, int V,
                        float *pv, int *pi, unsigned *ticket, int *am, float *ml,
                        hipStream_t st)
{
    if (M <= 1)
        launch_lm<NC, 1>(h, w, M, H, V, pv, pi, ticket, am, ml, st);
    else if (M <= 2)
        launch_lm<NC, 2>(h, w, M, H, V, pv, pi, ticket, am, ml, st);
    else if (M <= 4)
        launch_lm<NC, 4>(h, w, M, H, V, pv, pi, ticket, am, ml, st);
    else if (M <= 8)
        launch_lm<NC, 8>(h, w, M, H, V, pv, pi, ticket, am, ml, st);
    else
        launch_lm<NC, 16>(h, w, M, H, V, pv, pi, ticket, am, ml, st);
}

} // namespace mv

using namespace mv;

// Workspace: the header (ticket), [grid][M] fp32 best values, [grid][M]
// int32 best rows.
extern "C" size_t lmhead_argmax_workspace_bytes(int32_t M, int32_t V)
{
    if (M < 1 || M > kMaxM || V < 1)
        return 0;
    const size_t slots = (size_t)lm_grid(V) * (size_t)M;
    return kWsHeader + 2 * align_up(slots * 4, 256);
}

extern "C" moe_status_t lmhead_argmax(const uint16_t *h, const uint16_t *w_lm,
                                      int32_t M, int32_t H, int32_t V,
                                      int32_t *argmax, float *max_logit,
                                      void *workspace, size_t workspace_bytes,
                                      void *stream)
{
    if (!h || !w_lm || !argmax || !workspace)
        return MOE_ERR_NULL;
    if (M < 1 || H < 1 || V < 1)
        return MOE_ERR_SHAPE;
    if (M > kMaxM || H % 8 != 0 || H > kMaxDim)
        return MOE_ERR_UNSUPPORTED;
    if (!aligned16(h) || !aligned16(w_lm) || !aligned4(argmax) ||
        (max_logit && !aligned4(max_logit)) || !aligned16(workspace))
        return MOE_ERR_ALIGN;
    if (workspace_bytes < lmhead_argmax_workspace_bytes(M, V))
        return MOE_ERR_WORKSPACE;
    const size_t slots = (size_t)lm_grid(V) * (size_t)M;
    unsigned *ticket = (unsigned *)workspace;
    float *pv = (float *)((char *)workspace + kWsHeader);
    int *pi = (int *)((char *)workspace + kWsHeader + align_up(slots * 4, 256));
    hipStream_t st = (hipStream_t)stream;
    const int need = (H / 8 + kWave - 1) / kWave;
    if (need <= 1)
        launch_lm_m<1>(h, w_lm, M, H, V, pv, pi, ticket, argmax, max_logit, st);
    else if (need <= 2)
        launch_lm_m<2>(h, w_lm, M, H, V, pv, pi, ticket, argmax, max_logit, st);
    else if (need <= 4)
        launch_lm_m<4>(h, w_lm, M, H, V, pv, pi, ticket, argmax, max_logit, st);
    else if (need <= 5)
        launch_lm_m<5>(h, w_lm, M, H, V, pv, pi, ticket, argmax, max_logit, st);
    else if (need <= 8)
        launch_lm_m<8>(h, w_lm, M, H, V, pv, pi, ticket, argmax, max_logit, st);
    else
        launch_lm_m<16>(h, w_lm, M, H, V, pv, pi, ticket, argmax, max_logit, st);
    return check_launch();
}
