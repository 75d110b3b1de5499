// expert.hip -- selected experts' SwiGLU FFN with weighted combine
// (moe_expert_ffn, moe_layer).
//
// MoE chain of the LMSYS post "Chasing the batch-1 floor: Ling-3.0-flash
// speculative decode on Blackwell", section "PDL: the latency floor of
// stacked small kernels" (grouping -> up-GEMM -> activation -> down-GEMM ->
// combine) with the two changes of section "Two fusions and a retune": the
// SwiGLU product is computed in fp32 inside the up projection and rounded
// once, and the combine is a single fp32 weighted sum per output.
//
// Work is cut into units = (column block v of <= 16 pairs sharing one
// expert, 16-row tile of the weight matrix). Workgroup b owns a contiguous
// run of units; its four wavefronts split the reduction axis K of every
// unit, each streaming its K range of the tile's 16 rows straight from HBM
// into a private LDS double buffer (non-temporal 128-bit direct-to-LDS
// loads, 1 KB per instruction, the next block always in flight, across unit
// boundaries too). The dot products run on the matrix cores
// (v_mfma_f32_16x16x32_bf16: A = 16 weight rows, B = the block's <= 16
// activation columns). The four partial tiles are summed through LDS in a
// fixed order, so results are bitwise reproducible and every pair's result
// depends only on its own token.
//
//   up       A = W_gate and W_up rows (two MFMAs share each B fragment),
//            B = x of the pairs' tokens (staged once per workgroup in LDS);
//            epilogue a = bf16(silu(g) * u) in fp32, one rounding.
//   down     A = W_down rows, B = the pairs' activations a (L2-resident,
//            fetched with the same direct-to-LDS loads);
//            epilogue y[pair, rows] = W_down a in fp32.
//   combine  out[t, r] = sum_j w[t,j] * y[(t,j), r], slots in order, fp32.
// Every workgroup rebuilds the pair grouping in LDS from topk_idx, which
// costs less than a separate launch.
#include "common.h"

#include <mutex>

namespace mv {

constexpr int kXWaves = 4;                          // wavefronts split K
constexpr int kXKB = 128;                           // K elements per block
constexpr int kXRowBytes = kXKB * 2;                // 256 B of a row per block
constexpr int kXRowsPerLd = 1024 / kXRowBytes;      // 4 rows per load instruction
constexpr int kXLoads = 16 / kXRowsPerLd;           // 4 loads per 16-row block
constexpr int kXLdStride = 1024 + 16;               // LDS bytes per load (padded)
constexpr int kXBuf = kXLoads * kXLdStride;         // one block of one matrix
constexpr int kXSteps = kXKB / 32;                  // MFMA steps per block
constexpr int kXThreads = kXWaves * kWave;
constexpr int kXGrid = 256;                         // one workgroup per CU
// static LDS (grouping + small arrays) stays below this margin
constexpr int kXLdsDynMax = 160 * 1024 - 8 * 1024;

static_assert(sizeof(Groups) + 64 <= 8 * 1024, "static LDS margin");

struct UnitRange {
    int u0, u1;       // this workgroup's units
    int kb0, kb1;     // this wavefront's K blocks
};

__device__ inline UnitRange unit_range(int nunits, int nkb)
{
    UnitRange r;
    const int per = (nunits + gridDim.x - 1) / gridDim.x;
    r.u0 = min(nunits, (int)blockIdx.x * per);
    r.u1 = min(nunits, r.u0 + per);
    const int wave = threadIdx.x / kWave;
    const int kper = (nkb + kXWaves - 1) / kXWaves;
    r.kb0 = min(nkb, wave * kper);
    r.kb1 = min(nkb, r.kb0 + kper);
    return r;
}

// Slot of this lane in a 16-row block load: row lrow of the four rows an
// instruction covers, 16-byte chunk lcol of that row's 256-byte run.
struct LdSlot {
    int lrow, lcol;
};
__device__ __forceinline__ LdSlot ld_slot(int lane)
{
    return LdSlot{lane / (kWave / kXRowsPerLd), lane % (kWave / kXRowsPerLd)};
}
// LDS byte offset of the A fragment of lane (row j, K group g) in a block
__device__ __forceinline__ int a_frag_off(int j, int g)
{
    return (j / kXRowsPerLd) * kXLdStride + (j % kXRowsPerLd) * kXRowBytes + g * 16;
}

// Issue the direct-to-LDS loads of one 16-row block of a [rows, K] matrix:
// rows row0 .. row0+15 (clamped to nrows-1), K block kb (chunks clamped to
// the row). Four instructions, 1 KB each.
__device__ __forceinline__ void issue_block(const u32x4 *__restrict__ base, int row0,
                                            int nrows, int nch, int kb, LdSlot sl,
                                            unsigned char *buf)
{
    int c = kb * (kXKB / 8) + sl.lcol;
    c = c < nch ? c : nch - 1;
#pragma unroll
    for (int q = 0; q < kXLoads; ++q) {
        int row = row0 + q * kXRowsPerLd + sl.lrow;
        row = row < nrows ? row : nrows - 1;
        load_lds16(base + (size_t)row * nch + c, buf + q * kXLdStride);
    }
}

// ------------------------------------------------------------------- up
__global__ __launch_bounds__(kXThreads) void expert_up_kernel(
    const u32x4 *__restrict__ x, const int *__restrict__ topk_idx,
    const u32x4 *__restrict__ wg, const u32x4 *__restrict__ wu, int M, int H,
    int I, int E, int k, uint16_t *__restrict__ act)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ Groups g;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nch = H / 8;
    const int nkb = (H + kXKB - 1) / kXKB;
    const int xs = nkb * (kXKB / 8) + 1;                 // padded x row, chunks
    const size_t xbytes = align_up((size_t)M * xs * 16, 256);
    u32x4 *s_x = (u32x4 *)smem;
    unsigned char *wbuf = smem + xbytes + wave * 4 * kXBuf;   // [2 bufs][gate, up]
    float *red = (float *)(smem + xbytes + kXWaves * 4 * kXBuf); // [3][64][8]

    for (int i = threadIdx.x; i < M * xs; i += blockDim.x) {
        const int t = i / xs, c = i % xs;
        s_x[i] = (c < nch) ? x[(size_t)t * nch + c] : u32x4{0, 0, 0, 0};
    }
    build_groups(topk_idx, M * k, E, g);                 // ends with a barrier

    const int TI = (I + 15) / 16;
    const UnitRange ur = unit_range(g.DV * TI, nkb);
    const LdSlot sl = ld_slot(lane);
    const int j = lane & 15, gq = lane >> 4;
    const int aoff = a_frag_off(j, gq);

    auto issue = [&](int u, int kb, int b) {
        const int v = u / TI, tile = u % TI;
        const size_t eoff = (size_t)g.vexp[v] * I;
        unsigned char *bb = wbuf + b * 2 * kXBuf;
        issue_block(wg + eoff * nch, tile * 16, I, nch, kb, sl, bb);
        issue_block(wu + eoff * nch, tile * 16, I, nch, kb, sl, bb + kXBuf);
    };

    int b = 0;
    const bool has_k = ur.kb0 < ur.kb1;
    if (has_k && ur.u0 < ur.u1)
        issue(ur.u0, ur.kb0, 0);
    for (int u = ur.u0; u < ur.u1; ++u) {
        const int v = u / TI, tile = u % TI;
        const int npair = g.vcnt[v];
        const bool col_ok = j < npair;
        const int p = col_ok ? g.sorted[g.vbeg[v] + j] : 0;
        const u32x4 *xrow = s_x + (p / k) * xs + gq;
        f32x4 ag = {0.0f, 0.0f, 0.0f, 0.0f}, au = ag;
        for (int kb = ur.kb0; kb < ur.kb1; ++kb) {
            // prefetch the next block of this wavefront's sequence
            const bool last_kb = kb + 1 == ur.kb1;
            const int nu = last_kb ? u + 1 : u;
            const int nkbi = last_kb ? ur.kb0 : kb + 1;
            if (nu < ur.u1) {
                issue(nu, nkbi, b ^ 1);
                wait_vmcnt<2 * kXLoads>();
            } else {
                wait_vmcnt<0>();
            }
            const unsigned char *bg = wbuf + b * 2 * kXBuf + aoff;
#pragma unroll
            for (int s = 0; s < kXSteps; ++s) {
                u32x4 xv = xrow[kb * (kXKB / 8) + 4 * s];
                if (!col_ok)
                    xv = u32x4{0, 0, 0, 0};
                ag = mfma_bf16(*(const MV_LDS u32x4 *)(bg + s * 64), xv, ag);
                au = mfma_bf16(*(const MV_LDS u32x4 *)(bg + kXBuf + s * 64), xv, au);
            }
            b ^= 1;
        }
        // sum the four K partials in wavefront order, then SwiGLU
        if (wave > 0) {
            float *rp = red + ((wave - 1) * kWave + lane) * 8;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                rp[r] = ag[r];
                rp[4 + r] = au[r];
            }
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int w = 1; w < kXWaves; ++w) {
                const float *rp = red + ((w - 1) * kWave + lane) * 8;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    ag[r] += rp[r];
                    au[r] += rp[4 + r];
                }
            }
            if (col_ok) {
                // rows 4gq .. 4gq+3 of the tile for pair p
                const int row0 = tile * 16 + 4 * gq;
                uint32_t h[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float gv = ag[r];
                    const float a = gv / (1.0f + expf(-gv)) * au[r];
                    h[r] = f32_to_bf16_rne(a);
                }
                uint16_t *dst = act + (size_t)p * I + row0;
                if (row0 + 3 < I && (I % 4) == 0) {
                    *(uint2 *)dst = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
                } else {
                    for (int r = 0; r < 4; ++r)
                        if (row0 + r < I)
                            dst[r] = (uint16_t)h[r];
                }
            }
        }
        __syncthreads();
    }
}

// ----------------------------------------------------------------- down
constexpr int kXBBuf = kXSteps * 1024;              // B fragments of one block

__global__ __launch_bounds__(kXThreads) void expert_down_kernel(
    const u32x4 *__restrict__ act, const int *__restrict__ topk_idx,
    const u32x4 *__restrict__ wd, int M, int H, int I, int E, int k,
    float *__restrict__ y)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ Groups g;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nch = I / 8;                               // K = I here
    const int nkb = (I + kXKB - 1) / kXKB;
    unsigned char *wbuf = smem + wave * 2 * kXBuf;                    // A blocks
    unsigned char *bbuf = smem + kXWaves * 2 * kXBuf + wave * 2 * kXBBuf;  // B blocks
    float *red = (float *)(smem + kXWaves * 2 * (kXBuf + kXBBuf));    // [3][64][4]

    build_groups(topk_idx, M * k, E, g);

    const int TH = (H + 15) / 16;
    const UnitRange ur = unit_range(g.DV * TH, nkb);
    const LdSlot sl = ld_slot(lane);
    const int j = lane & 15, gq = lane >> 4;
    const int aoff = a_frag_off(j, gq);

    // A: 16 rows of W_down[e]; B: lane (j, gq) fetches the activation chunks
    // of pair j for its K group, one 1 KB load per MFMA step, landing in lane
    // order so that each lane later reads back exactly its own fragment
    auto issue = [&](int u, int kb, int b) {
        const int v = u / TH, tile = u % TH;
        issue_block(wd + (size_t)g.vexp[v] * H * nch, tile * 16, H, nch, kb, sl,
                    wbuf + b * kXBuf);
        const int p = j < g.vcnt[v] ? g.sorted[g.vbeg[v] + j] : 0;
#pragma unroll
        for (int s = 0; s < kXSteps; ++s) {
            int c = kb * (kXKB / 8) + 4 * s + gq;
            c = c < nch ? c : nch - 1;
            load_lds16(act + (size_t)p * nch + c, bbuf + b * kXBBuf + s * 1024);
        }
    };

    int b = 0;
    const bool has_k = ur.kb0 < ur.kb1;
    if (has_k && ur.u0 < ur.u1)
        issue(ur.u0, ur.kb0, 0);
    for (int u = ur.u0; u < ur.u1; ++u) {
        const int v = u / TH, tile = u % TH;
        const bool col_ok = j < g.vcnt[v];
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int kb = ur.kb0; kb < ur.kb1; ++kb) {
            const bool last_kb = kb + 1 == ur.kb1;
            const int nu = last_kb ? u + 1 : u;
            const int nkbi = last_kb ? ur.kb0 : kb + 1;
            if (nu < ur.u1) {
                issue(nu, nkbi, b ^ 1);
                wait_vmcnt<kXLoads + kXSteps>();
            } else {
                wait_vmcnt<0>();
            }
            const unsigned char *ba = wbuf + b * kXBuf + aoff;
            const unsigned char *bb = bbuf + b * kXBBuf + lane * 16;
#pragma unroll
            for (int s = 0; s < kXSteps; ++s) {
                u32x4 bv = *(const MV_LDS u32x4 *)(bb + s * 1024);
                if (!col_ok || kb * (kXKB / 8) + 4 * s + gq >= nch)
                    bv = u32x4{0, 0, 0, 0};
                acc = mfma_bf16(*(const MV_LDS u32x4 *)(ba + s * 64), bv, acc);
            }
            b ^= 1;
        }
        if (wave > 0) {
            float *rp = red + ((wave - 1) * kWave + lane) * 4;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                rp[r] = acc[r];
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int w = 1; w < kXWaves; ++w) {
                const float *rp = red + ((w - 1) * kWave + lane) * 4;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[r] += rp[r];
            }
            if (col_ok) {
                const int p = g.sorted[g.vbeg[v] + j];
                const int row0 = tile * 16 + 4 * gq;
                float *dst = y + (size_t)p * H + row0;
                if (row0 + 3 < H && (H % 4) == 0) {
                    *(float4 *)dst = make_float4(acc[0], acc[1], acc[2], acc[3]);
                } else {
                    for (int r = 0; r < 4; ++r)
                        if (row0 + r < H)
                            dst[r] = acc[r];
                }
            }
        }
        __syncthreads();
    }
}

// -------------------------------------------------------------- combine
__global__ __launch_bounds__(256) void expert_combine_kernel(
    const float *__restrict__ y, const int *__restrict__ topk_idx,
    const float *__restrict__ topk_w, int M, int H, int E, int k,
    float *__restrict__ out)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= M * H)
        return;
    const int t = i / H, r = i % H;
    float s = 0.0f;
    for (int jj = 0; jj < k; ++jj) {
        const int p = t * k + jj;
        const int e = topk_idx[p];
        if (e >= 0 && e < E)
            s = fmaf(topk_w[p], y[(size_t)p * H + r], s);
    }
    out[i] = s;
}

// ------------------------------------------------------------------ host

static size_t up_lds_bytes(int M, int H)
{
    const int nkb = (H + kXKB - 1) / kXKB;
    return align_up((size_t)M * (nkb * (kXKB / 8) + 1) * 16, 256) +
           (size_t)kXWaves * 4 * kXBuf + (size_t)(kXWaves - 1) * kWave * 8 * 4;
}
static size_t down_lds_bytes()
{
    return (size_t)kXWaves * 2 * (kXBuf + kXBBuf) + (size_t)(kXWaves - 1) * kWave * 4 * 4;
}

// Workspace: the header, the [M*k, I] bf16 activations, the [M*k, H] fp32
// per-pair down projections.
static size_t ffn_act_bytes(int32_t M, int32_t I, int32_t k)
{
    return align_up((size_t)M * k * I * sizeof(uint16_t), 256);
}
static size_t ffn_ws_bytes(int32_t M, int32_t H, int32_t I, int32_t k)
{
    return kWsHeader + ffn_act_bytes(M, I, k) + align_up((size_t)M * k * H * sizeof(float), 256);
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
    if (I % 8 != 0 || I > kMaxDim || up_lds_bytes(M, H) > (size_t)kXLdsDynMax)
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
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute((const void *)expert_up_kernel,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, kXLdsDynMax);
    });
    if (attr != hipSuccess)
        return MOE_ERR_LAUNCH;
    uint16_t *act = (uint16_t *)((char *)ws + kWsHeader);
    float *y = (float *)((char *)ws + kWsHeader + ffn_act_bytes(M, I, k));
    hipLaunchKernelGGL(expert_up_kernel, dim3(kXGrid), dim3(kXThreads),
                       up_lds_bytes(M, H), st, (const u32x4 *)x, topk_idx,
                       (const u32x4 *)w_gate, (const u32x4 *)w_up, M, H, I, E, k, act);
    moe_status_t s = check_launch();
    if (s != MOE_OK)
        return s;
    hipLaunchKernelGGL(expert_down_kernel, dim3(kXGrid), dim3(kXThreads), down_lds_bytes(),
                       st, (const u32x4 *)act, topk_idx, (const u32x4 *)w_down, M, H, I,
                       E, k, y);
    s = check_launch();
    if (s != MOE_OK)
        return s;
    const int n = M * H;
    hipLaunchKernelGGL(expert_combine_kernel, dim3((n + 255) / 256), dim3(256), 0, st, y,
                       topk_idx, topk_w, M, H, E, k, out);
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
    return ffn_ws_bytes(M, H, I, k);
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
