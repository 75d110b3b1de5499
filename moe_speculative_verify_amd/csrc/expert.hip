// expert.hip -- selected experts' SwiGLU FFN with weighted combine
// (moe_expert_ffn, moe_layer).
//
// MoE chain of the LMSYS post "Chasing the batch-1 floor: Ling-3.0-flash
// speculative decode on Blackwell", section "PDL: the latency floor of
// stacked small kernels" (grouping -> up-GEMM -> activation -> down-GEMM ->
// combine) with the two changes of section "Two fusions and a retune": the
// SwiGLU product is computed in fp32 inside the up projection and rounded
// once, and the combine is a single fp32 weighted sum.
//
// At batch 1 every selected expert serves one to sixteen tokens, so each
// projection is a GEMV bound by the cold weight read. Two kernels:
//   up    every workgroup rebuilds the pair grouping in LDS from topk_idx
//         (cheaper than a launch), then streams an equal share of the
//         D * I (gate row, up row) pairs of the D distinct experts with
//         128-bit loads; each wavefront keeps RB row pairs in flight,
//         reduces one fp32 dot per token and row, and writes
//         a = bf16(silu(g) * u) per (pair, i).
//   down  workgroup b owns rows [r0, r1) of the output for every expert:
//         its wavefronts stream those rows of W_down for the distinct
//         experts, dot them with the activations of each pair, and the
//         workgroup then forms out[t, r] = sum_j w[t,j] y[(t,j), r] in slot
//         order. No float atomics: results are bitwise reproducible and a
//         token's result does not depend on the other tokens.
#include "common.h"

namespace mv {

constexpr int kUpThreads = 256;
constexpr int kDownThreads = 256;

// ------------------------------------------------------------------ up
template <int NC, int RB>  // NC chunks per lane of H; RB row pairs in flight
__global__ __launch_bounds__(kUpThreads) void expert_up_kernel(
    const u32x4 *__restrict__ x, const int *__restrict__ topk_idx,
    const u32x4 *__restrict__ wg, const u32x4 *__restrict__ wu, int M, int H,
    int I, int E, int k, uint16_t *__restrict__ act)
{
    __shared__ Groups g;
    build_groups(topk_idx, M * k, E, g);

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwave = blockDim.x / kWave;
    const int nchunk = H / 8;

    // equal shares of the D*I row pairs, in whole groups of RB (RB divides I,
    // so a group never straddles two experts)
    const long ngroups = (long)g.D * (I / RB);
    const long per_wg = (ngroups + gridDim.x - 1) / gridDim.x;
    const long b0 = (long)blockIdx.x * per_wg;
    const long b1 = min(ngroups, b0 + per_wg);
    const long per_w = (b1 - b0 + nwave - 1) / nwave;
    const long w0 = b0 + (long)wave * per_w;
    const long w1 = min(b1, w0 + per_w);

    for (long grp = w0; grp < w1; ++grp) {
        const long q = grp * RB;                 // first row pair
        const int d = (int)(q / I);
        const int i0 = (int)(q % I);
        const int e = g.dexp[d];
        const size_t row0 = ((size_t)e * I + i0) * nchunk;

        u32x4 G[RB][NC], U[RB][NC];
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int ci = lane + kWave * c;
                if (ci < nchunk) {
                    G[b][c] = load_stream(wg + row0 + (size_t)b * nchunk + ci);
                    U[b][c] = load_stream(wu + row0 + (size_t)b * nchunk + ci);
                } else {
                    G[b][c] = U[b][c] = u32x4{0, 0, 0, 0};
                }
            }

        for (int s = g.doff[d]; s < g.doff[d + 1]; ++s) {
            const int p = g.sorted[s];
            const int t = p / k;
            u32x4 xv[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int ci = lane + kWave * c;
                xv[c] = (ci < nchunk) ? x[(size_t)t * nchunk + ci] : u32x4{0, 0, 0, 0};
            }
            float ag[RB], au[RB];
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                float sg = 0.0f, su = 0.0f;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    sg = dot8_bf16(G[b][c], xv[c], sg);
                    su = dot8_bf16(U[b][c], xv[c], su);
                }
                ag[b] = wave_sum(sg);
                au[b] = wave_sum(su);
            }
            if (lane < RB) {
                // SwiGLU in fp32, one rounding of the product to bf16
                float gv = ag[0], uv = au[0];
#pragma unroll
                for (int b = 1; b < RB; ++b)
                    if (lane == b) {
                        gv = ag[b];
                        uv = au[b];
                    }
                const float a = gv / (1.0f + expf(-gv)) * uv;
                act[(size_t)p * I + i0 + lane] = (uint16_t)f32_to_bf16_rne(a);
            }
        }
    }
}

// ---------------------------------------------------------------- down
template <int NC, int RB>  // NC chunks per lane of I; RB rows in flight
__global__ __launch_bounds__(kDownThreads) void expert_down_kernel(
    const u32x4 *__restrict__ act, const int *__restrict__ topk_idx,
    const float *__restrict__ topk_w, const u32x4 *__restrict__ wd, int M,
    int H, int I, int E, int k, int rows_per_wg, float *__restrict__ out)
{
    __shared__ Groups g;
    extern __shared__ float s_y[];               // [NP][rows_per_wg]
    build_groups(topk_idx, M * k, E, g);

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwave = blockDim.x / kWave;
    const int nchunk = I / 8;
    const int r0 = blockIdx.x * rows_per_wg;
    const int r1 = min(H, r0 + rows_per_wg);
    const int nr = r1 - r0;
    if (nr <= 0)
        return;

    for (int d = wave; d < g.D; d += nwave) {
        const int e = g.dexp[d];
        for (int r = r0; r < r1; r += RB) {
            u32x4 W[RB][NC];
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int ci = lane + kWave * c;
                    W[b][c] = (r + b < r1 && ci < nchunk)
                                  ? load_stream(wd + ((size_t)e * H + r + b) * nchunk + ci)
                                  : u32x4{0, 0, 0, 0};
                }
            for (int s = g.doff[d]; s < g.doff[d + 1]; ++s) {
                const int p = g.sorted[s];
                u32x4 av[NC];
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int ci = lane + kWave * c;
                    av[c] = (ci < nchunk) ? act[(size_t)p * nchunk + ci] : u32x4{0, 0, 0, 0};
                }
#pragma unroll
                for (int b = 0; b < RB; ++b) {
                    float acc = 0.0f;
#pragma unroll
                    for (int c = 0; c < NC; ++c)
                        acc = dot8_bf16(W[b][c], av[c], acc);
                    acc = wave_sum(acc);
                    if (lane == 0 && r + b < r1)
                        s_y[p * rows_per_wg + (r + b - r0)] = acc;
                }
            }
        }
    }
    __syncthreads();

    // weighted combine, slots in order, fp32
    for (int i = threadIdx.x; i < M * nr; i += blockDim.x) {
        const int t = i / nr, rr = i % nr;
        float sum = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int p = t * k + j;
            if (g.e[p] >= 0)
                sum = fmaf(topk_w[p], s_y[p * rows_per_wg + rr], sum);
        }
        out[(size_t)t * H + r0 + rr] = sum;
    }
}

// ------------------------------------------------------------------ host

static int chunks_per_lane(int n) { return (n / 8 + kWave - 1) / kWave; }

// Grid sizes: the up share is split evenly on the device once D is known;
// the down rows are split over a fixed number of workgroups.
constexpr int kUpGrid = 512;
constexpr int kDownGrid = 256;

template <int NC>
static void launch_up_nc(const uint16_t *x, const int *idx, const uint16_t *wg,
                         const uint16_t *wu, int M, int H, int I, int E, int k,
                         uint16_t *act, hipStream_t st)
{
    if (NC <= 8 && I % 2 == 0)
        hipLaunchKernelGGL((expert_up_kernel<NC, (NC <= 8 ? 2 : 1)>), dim3(kUpGrid),
                           dim3(kUpThreads), 0, st, (const u32x4 *)x, idx,
                           (const u32x4 *)wg, (const u32x4 *)wu, M, H, I, E, k, act);
    else
        hipLaunchKernelGGL((expert_up_kernel<NC, 1>), dim3(kUpGrid), dim3(kUpThreads),
                           0, st, (const u32x4 *)x, idx, (const u32x4 *)wg,
                           (const u32x4 *)wu, M, H, I, E, k, act);
}

static void launch_up(const uint16_t *x, const int *idx, const uint16_t *wg,
                      const uint16_t *wu, int M, int H, int I, int E, int k,
                      uint16_t *act, hipStream_t st)
{
    const int need = chunks_per_lane(H);
    if (need <= 1)
        launch_up_nc<1>(x, idx, wg, wu, M, H, I, E, k, act, st);
    else if (need <= 2)
        launch_up_nc<2>(x, idx, wg, wu, M, H, I, E, k, act, st);
    else if (need <= 4)
        launch_up_nc<4>(x, idx, wg, wu, M, H, I, E, k, act, st);
    else if (need <= 5)
        launch_up_nc<5>(x, idx, wg, wu, M, H, I, E, k, act, st);
    else if (need <= 8)
        launch_up_nc<8>(x, idx, wg, wu, M, H, I, E, k, act, st);
    else
        launch_up_nc<16>(x, idx, wg, wu, M, H, I, E, k, act, st);
}

template <int NC>
static void launch_down_nc(const uint16_t *act, const int *idx, const float *tw,
                           const uint16_t *wd, int M, int H, int I, int E, int k,
                           float *out, hipStream_t st)
{
    const int rows = (H + kDownGrid - 1) / kDownGrid;
    const int grid = (H + rows - 1) / rows;
    const size_t lds = (size_t)M * k * rows * sizeof(float);
    if (rows % 5 == 0)
        hipLaunchKernelGGL((expert_down_kernel<NC, 5>), dim3(grid), dim3(kDownThreads),
                           lds, st, (const u32x4 *)act, idx, tw, (const u32x4 *)wd,
                           M, H, I, E, k, rows, out);
    else if (rows % 4 == 0)
        hipLaunchKernelGGL((expert_down_kernel<NC, 4>), dim3(grid), dim3(kDownThreads),
                           lds, st, (const u32x4 *)act, idx, tw, (const u32x4 *)wd,
                           M, H, I, E, k, rows, out);
    else
        hipLaunchKernelGGL((expert_down_kernel<NC, 2>), dim3(grid), dim3(kDownThreads),
                           lds, st, (const u32x4 *)act, idx, tw, (const u32x4 *)wd,
                           M, H, I, E, k, rows, out);
}

static void launch_down(const uint16_t *act, const int *idx, const float *tw,
                        const uint16_t *wd, int M, int H, int I, int E, int k,
                        float *out, hipStream_t st)
{
    const int need = chunks_per_lane(I);
    if (need <= 1)
        launch_down_nc<1>(act, idx, tw, wd, M, H, I, E, k, out, st);
    else if (need <= 2)
        launch_down_nc<2>(act, idx, tw, wd, M, H, I, E, k, out, st);
    else if (need <= 4)
        launch_down_nc<4>(act, idx, tw, wd, M, H, I, E, k, out, st);
    else if (need <= 8)
        launch_down_nc<8>(act, idx, tw, wd, M, H, I, E, k, out, st);
    else
        launch_down_nc<16>(act, idx, tw, wd, M, H, I, E, k, out, st);
}

// Workspace: the header, then the [M*k, I] bf16 SwiGLU activations.
static size_t ffn_ws_bytes(int32_t M, int32_t I, int32_t k)
{
    return kWsHeader + align_up((size_t)M * k * I * sizeof(uint16_t), 256);
}

static moe_status_t ffn_check(const uint16_t *x, const int32_t *topk_idx,
                              const float *topk_w, const uint16_t *w_gate,
                              const uint16_t *w_up, const uint16_t *w_down,
                              int32_t M, int32_t H, int32_t I, int32_t E,
                              int32_t k, const float *out)
{
    if (!x || !topk_idx || !topk_w || !w_gate || !w_up || !w_down || !out)
        return MOE_ERR_NULL;
    moe_status_t s = check_moe_shape(M, H, E, k);
    if (s != MOE_OK)
        return s;
    if (I < 1)
        return MOE_ERR_SHAPE;
    if (I % 8 != 0 || I > kMaxDim)
        return MOE_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) ||
        !aligned16(w_down) || !aligned4(topk_idx) || !aligned4(topk_w) ||
        !aligned4(out))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

static moe_status_t ffn_enqueue(const uint16_t *x, const int32_t *topk_idx,
                                const float *topk_w, const uint16_t *w_gate,
                                const uint16_t *w_up, const uint16_t *w_down,
                                int32_t M, int32_t H, int32_t I, int32_t E,
                                int32_t k, float *out, void *ws, hipStream_t st)
{
    uint16_t *act = (uint16_t *)((char *)ws + kWsHeader);
    launch_up(x, topk_idx, w_gate, w_up, M, H, I, E, k, act, st);
    moe_status_t s = check_launch();
    if (s != MOE_OK)
        return s;
    launch_down(act, topk_idx, topk_w, w_down, M, H, I, E, k, out, st);
    return check_launch();
}

// route.hip
moe_status_t route_check(const uint16_t *x, const uint16_t *w_router,
                         const float *bias, int32_t M, int32_t H, int32_t E,
                         int32_t k, const int32_t *topk_idx, const float *topk_w,
                         const float *logits);
moe_status_t route_enqueue(const uint16_t *x, const uint16_t *w_router,
                           const float *bias, int32_t M, int32_t H, int32_t E,
                           int32_t k, int32_t *topk_idx, float *topk_w,
                           float *logits, void *ws, hipStream_t st);

} // namespace mv

using namespace mv;

extern "C" size_t moe_expert_ffn_workspace_bytes(int32_t M, int32_t H, int32_t I,
                                                 int32_t E, int32_t k)
{
    if (check_moe_shape(M, H, E, k) != MOE_OK || I < 8 || I % 8 || I > kMaxDim)
        return 0;
    return ffn_ws_bytes(M, I, k);
}

extern "C" moe_status_t moe_expert_ffn(const uint16_t *x, const int32_t *topk_idx,
                                       const float *topk_w, const uint16_t *w_gate,
                                       const uint16_t *w_up, const uint16_t *w_down,
                                       int32_t M, int32_t H, int32_t I, int32_t E,
                                       int32_t k, float *out, void *workspace,
                                       size_t workspace_bytes, void *stream)
{
    moe_status_t s = ffn_check(x, topk_idx, topk_w, w_gate, w_up, w_down, M, H, I,
                               E, k, out);
    if (s != MOE_OK)
        return s;
    if (!workspace)
        return MOE_ERR_NULL;
    if (!aligned16(workspace))
        return MOE_ERR_ALIGN;
    if (workspace_bytes < moe_expert_ffn_workspace_bytes(M, H, I, E, k))
        return MOE_ERR_WORKSPACE;
    return ffn_enqueue(x, topk_idx, topk_w, w_gate, w_up, w_down, M, H, I, E, k,
                       out, workspace, (hipStream_t)stream);
}

extern "C" size_t moe_layer_workspace_bytes(int32_t M, int32_t H, int32_t I,
                                            int32_t E, int32_t k)
{
    // the route's layout (header + logits) followed by the FFN's data part
    const size_t f = moe_expert_ffn_workspace_bytes(M, H, I, E, k);
    const size_t r = moe_route_workspace_bytes(M, E);
    if (!f || !r)
        return 0;
    return r + (f - kWsHeader);
}

extern "C" moe_status_t moe_layer(const uint16_t *x, const uint16_t *w_router,
                                  const float *bias, const uint16_t *w_gate,
                                  const uint16_t *w_up, const uint16_t *w_down,
                                  int32_t M, int32_t H, int32_t I, int32_t E,
                                  int32_t k, int32_t *topk_idx, float *topk_w,
                                  float *out, void *workspace,
                                  size_t workspace_bytes, void *stream)
{
    moe_status_t s = route_check(x, w_router, bias, M, H, E, k, topk_idx, topk_w,
                                 nullptr);
    if (s != MOE_OK)
        return s;
    s = ffn_check(x, topk_idx, topk_w, w_gate, w_up, w_down, M, H, I, E, k, out);
    if (s != MOE_OK)
        return s;
    if (!workspace)
        return MOE_ERR_NULL;
    if (!aligned16(workspace))
        return MOE_ERR_ALIGN;
    if (workspace_bytes < moe_layer_workspace_bytes(M, H, I, E, k))
        return MOE_ERR_WORKSPACE;
    // the FFN's data part starts where the route's ends; its header slot
    // overlaps the route's logits, which the FFN never reads
    const size_t r = moe_route_workspace_bytes(M, E);
    hipStream_t st = (hipStream_t)stream;
    s = route_enqueue(x, w_router, bias, M, H, E, k, topk_idx, topk_w, nullptr,
                      workspace, st);
    if (s != MOE_OK)
        return s;
    return ffn_enqueue(x, topk_idx, topk_w, w_gate, w_up, w_down, M, H, I, E, k,
                       out, (char *)workspace + r - kWsHeader, st);
}
