// lmhead.hip -- lm_head GEMV fused with the greedy argmax (lmhead_argmax).
//
// The LMSYS post "Chasing the batch-1 floor: Ling-3.0-flash speculative
// decode on Blackwell" runs the lm_head in bf16 because at batch 1 it is a
// pure weight read (section "bf16 router gate and lm_head"); its logits feed
// the greedy verdict inside the verify step (section "The shape of a
// single-request step", Fig. 3).
//
// Design (gfx950):
//   - The vocabulary is cut into 16-row tiles, dealt round-robin: wavefront w
//     of workgroup b (of G) takes tiles b + G (w + 4 i), i = 0, 1, ..., so
//     at any moment the whole chip streams one window of neighbouring tiles
//     (the access order of the fastest plain read measured on this part).
//   - A wavefront streams its tile K-block by K-block (KB elements of each of
//     the 16 rows) straight from HBM into its own LDS ring (two slots, a
//     third where the LDS has room) with non-temporal 128-bit direct-to-LDS
//     loads: every load instruction reads 1 KB made of two 512-byte row
//     runs, the access pattern that reaches the HBM roofline, and the next
//     block is in flight while the current one is consumed (the next two in
//     the wavefront's last tile, when it has a third slot).
//   - The dot products run on the matrix cores: v_mfma_f32_16x16x32_bf16
//     with A = 16 weight rows (from LDS) and B = the M <= 16 hidden states
//     (staged once per workgroup in LDS, zero columns beyond M). One MFMA
//     covers 1 KB of weights; no cross-lane reductions are needed.
//   - Each lane keeps a running (max, first index) for its token; the
//     workgroup's best per token becomes a 64-bit key (order-preserving
//     value bits << 32 | ~index, so the largest value and then the lowest
//     index win) stored in the workgroup's own slot of the workspace. A
//     second kernel of one workgroup, launched behind it on the same
//     stream, takes each token's maximum over the slots and decodes it:
//     the kernel boundary orders every slot's store before the merge's
//     loads, so no workgroup pays for a device-scope release or acquire
//     (a last-workgroup hand-off inside the kernel, counted with
//     agent-scope releases and acquired by the last arrival, measured
//     6-7 us slower per call: each release writes back an XCD's L2 while
//     the other workgroups there still stream). Every slot is written
//     before it is read, so nothing past the header needs to be zero, and
//     the header's counters are not used.
//   - fp8 weights (lmhead_argmax_fp8, lmhead_greedy_verify_fp8): OCP E4M3
//     codes with one fp32 scale per vocabulary row. A block is still 512
//     bytes of each of the 16 rows (now 512 columns), staged the same way;
//     each MFMA step reads the lane's eight codes from LDS, widens them to
//     bf16 (exact), and the row scales multiply the fp32 tile before the
//     argmax.
//   - lmhead_greedy_verify: the same two kernels; the merge then takes the
//     greedy verdict of the verify chain from the decoded tokens (section
//     "The shape of a single-request step": the verdict is part of the
//     verify step and stays on the device).
#include "common.h"

#include <mutex>

namespace mv {

constexpr int kLmWaves = 4;
// one workgroup per CU: the LDS footprint allows no more
constexpr int kLmGridTarget = 256;
static_assert(kMaxM % kLmWaves == 0 && kLmGridTarget % kWave == 0, "key slots per lane");
constexpr int kLmRowBytes = 512;                  // bytes of a row per block
constexpr int kLmRowsPerLd = 1024 / kLmRowBytes;  // rows per load instruction
constexpr int kLmLoads = 16 / kLmRowsPerLd;       // load instructions per block
constexpr int kLmLdStride = 1024 + 16;            // LDS bytes per load (padded)
constexpr int kLmBuf = kLmLoads * kLmLdStride;    // one block of a tile
constexpr int kLmRowCh = kLmRowBytes / 16;        // 16-byte chunks of a row per block
// K elements per block: 256 bf16 or 512 fp8 columns
constexpr int lm_kb(bool w8) { return w8 ? kLmRowBytes : kLmRowBytes / 2; }

__host__ __device__ static size_t lm_x_bytes(int M, int H, bool w8)
{
    const int KB = lm_kb(w8);
    const int nkb = (H + KB - 1) / KB;
    return align_up((size_t)M * (nkb * (KB / 8) + 1) * 16, 256);
}
static size_t lm_lds_bytes(int M, int H, bool w8, int nslot = 2)
{
    return lm_x_bytes(M, H, w8) + (size_t)kLmWaves * nslot * kLmBuf;
}

template <bool W8>
__global__ __launch_bounds__(kLmWaves * kWave) void lmhead_kernel(
    const u32x4 *__restrict__ h, const u32x4 *__restrict__ wl,
    const float *__restrict__ wscale, int M, int H,
    int V, unsigned long long *__restrict__ keys, int nslot)
{
    constexpr int KB = lm_kb(W8);
    constexpr int kLmSteps = KB / 32;                    // MFMA steps per block
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nch = H / 8;                               // bf16 chunks of an h row
    const int nwch = W8 ? H / 16 : nch;                  // 16-byte chunks of a weight row
    const int nkb = (H + KB - 1) / KB;
    const int xs = nkb * (KB / 8) + 1;                   // padded x row, chunks
    u32x4 *s_x = (u32x4 *)smem;
    unsigned char *wbuf = smem + lm_x_bytes(M, H, W8) + wave * nslot * kLmBuf;

    // hidden states into LDS with direct-to-LDS loads (all in flight at
    // once), K padding zeroed
    for (int i = threadIdx.x; i < M * (xs - nch); i += blockDim.x) {
        const int t = i / (xs - nch), c = nch + i % (xs - nch);
        s_x[t * xs + c] = u32x4{0, 0, 0, 0};
    }
    stage_rows_lds(h, M, nch, s_x, xs);
    wait_vmcnt<0>();
    __syncthreads();

    const int j = lane & 15;        // A row in the tile / B column = token
    const int g = lane >> 4;        // K group of 8 elements in an MFMA step
    const bool tok_ok = j < M;
    const u32x4 *xrow = s_x + (tok_ok ? j : 0) * xs + g;
    // this lane's slot in a load instruction: row lrow of the group of
    // rows the instruction covers, chunk lcol of that row's block
    const int lrow = lane / (kWave / kLmRowsPerLd);
    const int lcol = lane % (kWave / kLmRowsPerLd);
    // lane (j, g) reads row j's columns [32 s + 8 g, +8) of step s: 16 bytes
    // of bf16 or 8 bytes of fp8
    const int a_off = (j / kLmRowsPerLd) * kLmLdStride + (j % kLmRowsPerLd) * kLmRowBytes +
                      g * (W8 ? 8 : 16);

    const int ntiles = (V + 15) / 16;
    // running (max, first row) of this lane; kNoRow until its first row
    float bv = -INFINITY;
    int bi = kNoRow;

    // The ring runs across tiles: while a tile's last block is consumed, the
    // next tile's first block is already in flight, so every wavefront keeps
    // one block in flight from its first tile to its last. Where the LDS
    // holds a third slot per wavefront (nslot = 3), the last tile keeps two
    // blocks in flight: by then most wavefronts have finished and the HBM
    // has room, and a wavefront's single block in flight would set the pace
    // (paired: 0.9 us less per call at M = 6, 0.8 at M = 1; two blocks ahead
    // in every tile measured slower). Block n of the wavefront (counted over
    // its tiles) sits in slot n % nslot.
    auto tile_rows = [&](int tile, const u32x4 *(&rp)[kLmLoads]) {
#pragma unroll
        for (int q = 0; q < kLmLoads; ++q) {
            int row = tile * 16 + q * kLmRowsPerLd + lrow;
            row = row < V ? row : V - 1;                 // tail rows: valid memory, ignored
            rp[q] = wl + (size_t)row * nwch;
        }
    };
    auto issue = [&](const u32x4 *(&rp)[kLmLoads], int kb, int buf) {
        int c = kb * kLmRowCh + lcol;
        c = c < nwch ? c : nwch - 1;                     // K tail: valid memory, x is zero there
#pragma unroll
        for (int q = 0; q < kLmLoads; ++q)
            load_lds16(rp[q] + c, wbuf + buf * kLmBuf + q * kLmLdStride);
    };
    const int tstride = gridDim.x * kLmWaves;
    int tile = blockIdx.x + gridDim.x * wave;
    const u32x4 *rp[kLmLoads], *rpn[kLmLoads];
    int nblk = 0;                                        // blocks of this wavefront so far
    if (tile < ntiles) {
        tile_rows(tile, rp);
        issue(rp, 0, 0);
    }
    for (; tile < ntiles; tile += tstride) {
        const bool more = tile + tstride < ntiles;
        if (more)
            tile_rows(tile + tstride, rpn);
        // fp8: the scales of this lane's four tile rows, used after the K loop;
        // the tile's 16 scales are read with scalar loads (the tile index is
        // uniform), which the vector-memory waits of the ring do not count,
        // so using them never waits for the next tile's block in flight
        float rs[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if constexpr (W8) {
            float sc[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                sc[i] = wscale[min(tile * 16 + i, V - 1)];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                rs[r] = g == 0 ? sc[r] : g == 1 ? sc[4 + r] : g == 2 ? sc[8 + r] : sc[12 + r];
        }
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        const bool deep = !more && nslot == 3;           // the last tile: two blocks ahead
        for (int kb = 0; kb < nkb; ++kb) {
            const int b = (nblk + kb) % nslot;
            if (deep) {
                if (kb == 0 && kb + 1 < nkb)
                    issue(rp, kb + 1, (b + 1) % 3);
                if (kb + 2 < nkb)
                    issue(rp, kb + 2, (b + 2) % 3);
                if (kb + 2 < nkb)
                    wait_vmcnt<2 * kLmLoads>();          // block kb has landed
                else if (kb + 1 < nkb)
                    wait_vmcnt<kLmLoads>();
                else
                    wait_vmcnt<0>();
            } else if (kb + 1 < nkb) {
                issue(rp, kb + 1, (b + 1) % nslot);
                wait_vmcnt<kLmLoads>();                  // block kb has landed
            } else if (more) {
                issue(rpn, 0, (b + 1) % nslot);          // the next tile's first block
                wait_vmcnt<kLmLoads>();
            } else {
                wait_vmcnt<0>();
            }
            const unsigned char *ab = wbuf + b * kLmBuf + a_off;
#pragma unroll
            for (int s = 0; s < kLmSteps; ++s) {
                u32x4 a;
                if constexpr (W8) {
                    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                    const u32x2 q8 = *(const MV_LDS u32x2 *)(ab + s * 32);
                    a = e4m3x8_to_bf16(q8.x, q8.y);
                } else {
                    a = *(const MV_LDS u32x4 *)(ab + s * 64);
                }
                u32x4 x = xrow[kb * (KB / 8) + 4 * s];
                if (!tok_ok)
                    x = u32x4{0, 0, 0, 0};
                acc = mfma_bf16(a, x, acc);
            }
        }
        nblk += nkb;
        if (more) {
#pragma unroll
            for (int q = 0; q < kLmLoads; ++q)
                rp[q] = rpn[q];
        }
        if constexpr (W8) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[r] *= rs[r];
        }
        // rows 4g..4g+3 of the tile for token j, in ascending order
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = tile * 16 + 4 * g + r;
            if (row < V)
                argmax_take(bv, bi, acc[r], row);
        }
    }

    // the four lanes of token j (one per K group) hold interleaved rows
#pragma unroll
    for (int m = 16; m <= 32; m <<= 1) {
        const float ov = __shfl_xor(bv, m);
        const int oi = __shfl_xor(bi, m);
        argmax_merge(bv, bi, ov, oi);
    }
    __shared__ float s_v[kLmWaves][16];
    __shared__ int s_i[kLmWaves][16];
    if (g == 0) {
        s_v[wave][j] = bv;
        s_i[wave][j] = bi;
    }
    __syncthreads();
    if (threadIdx.x < M) {
        const int t = threadIdx.x;
        float best = s_v[0][t];
        int besti = s_i[0][t];
        for (int w = 1; w < kLmWaves; ++w)
            argmax_merge(best, besti, s_v[w][t], s_i[w][t]);
        keys[(size_t)blockIdx.x * M + t] = argmax_key(best, besti);
    }
}

// The merge of the G workgroups' keys, one workgroup of kLmWaves
// wavefronts: wavefront w takes tokens w, w + 4, ...; lane l reads slots
// l, l + 64, ... of each (every load in flight at once, clamped addresses),
// keeps the largest, and the largest key over the wavefront decodes the
// token. With tokens given, thread 0 then takes the greedy verdict.
__global__ __launch_bounds__(kLmWaves * kWave) void lmhead_merge_kernel(
    const unsigned long long *__restrict__ keys, int G, int M, int *__restrict__ argmax,
    float *__restrict__ max_logit, const int *__restrict__ tokens, int *__restrict__ accept)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    __shared__ int s_tok[kMaxM];
    constexpr int kTpw = kMaxM / kLmWaves;                // tokens per wavefront
    constexpr int kSpl = kLmGridTarget / kWave;           // slots per lane
    unsigned long long kv[kTpw][kSpl];
#pragma unroll
    for (int q = 0; q < kTpw; ++q) {
        const int t = min(wave + kLmWaves * q, M - 1);
#pragma unroll
        for (int sl = 0; sl < kSpl; ++sl)
            kv[q][sl] = keys[(size_t)min(lane + kWave * sl, G - 1) * M + t];
    }
#pragma unroll
    for (int q = 0; q < kTpw; ++q) {
        const int t = wave + kLmWaves * q;
        if (t >= M)                                      // uniform
            break;
        unsigned long long best = 0;
#pragma unroll
        for (int sl = 0; sl < kSpl; ++sl)
            best = kv[q][sl] > best ? kv[q][sl] : best;  // (clamped reads repeat a slot)
        const unsigned long long key = wave_max_key(best);
        if (lane == 0) {
            const int tok = argmax_key_row(key);
            argmax[t] = tok;
            s_tok[t] = tok;
            if (max_logit)
                max_logit[t] = f32_unorder((uint32_t)(key >> 32));
        }
    }
    if (tokens == nullptr)                               // uniform
        return;
    // Greedy verdict: drafted candidate i (chain position i >= 1) is
    // accepted while it equals the target's token after position i - 1;
    // the first rejection ends the prefix. accept = {n + 1, bonus token}.
    __syncthreads();
    if (threadIdx.x == 0) {
        int n = 0;
        while (n + 1 < M && tokens[n + 1] == s_tok[n])
            ++n;
        accept[0] = n + 1;
        accept[1] = s_tok[n];
    }
}


} // namespace mv

using namespace mv;

// Workspace: the header (not used here), then each workgroup's M 64-bit keys.
extern "C" size_t lmhead_argmax_workspace_bytes(int32_t M, int32_t V)
{
    if (M < 1 || M > kMaxM || V < 1)
        return 0;
    return kWsHeader + align_up((size_t)kLmGridTarget * M * 8, 256);
}

// The workgroups of the GEMV: one key slot each in the workspace.
static int lm_grid(int V)
{
    return min((V + 15) / 16, kLmGridTarget);
}

// Checks of the GEMV phase: w_lm bf16 rows, or fp8 codes when w8 (one
// scale per row); workspace: the keys, one M-key slot per workgroup.
static moe_status_t lm_check_keys(const uint16_t *h, const void *w_lm, const float *w_scale,
                                  bool w8, int32_t M, int32_t H, int32_t V,
                                  const void *workspace, size_t workspace_bytes)
{
    if (!h || !w_lm || !workspace || (w8 && !w_scale))
        return MOE_ERR_NULL;
    if (M < 1 || H < 1 || V < 1)
        return MOE_ERR_SHAPE;
    if (M > kMaxM || H % (w8 ? 16 : 8) != 0 || H > kMaxDim ||
        lm_lds_bytes(M, H, w8) > (size_t)kLdsDynMax)
        return MOE_ERR_UNSUPPORTED;
    if (w8 && !aligned4(w_scale))
        return MOE_ERR_ALIGN;
    if (!aligned16(h) || !aligned16(w_lm) || !aligned16(workspace))
        return MOE_ERR_ALIGN;
    if (workspace_bytes < lmhead_argmax_workspace_bytes(M, V))
        return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

// Checks of the merge phase (tokens and accept both given or both NULL).
static moe_status_t lm_check_merge(int32_t M, int32_t V, const int32_t *argmax,
                                   const float *max_logit, const int32_t *tokens,
                                   const int32_t *accept, const void *workspace,
                                   size_t workspace_bytes)
{
    if (!argmax || !workspace || (!tokens) != (!accept))
        return MOE_ERR_NULL;
    if (M < 1 || V < 1)
        return MOE_ERR_SHAPE;
    if (M > kMaxM)
        return MOE_ERR_UNSUPPORTED;
    if (!aligned4(argmax) || (max_logit && !aligned4(max_logit)) || !aligned16(workspace) ||
        (tokens && (!aligned4(tokens) || !aligned4(accept))))
        return MOE_ERR_ALIGN;
    if (workspace_bytes < lmhead_argmax_workspace_bytes(M, V))
        return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

// The GEMV phase: every workgroup's per-token winner as a 64-bit key in the
// workspace (arguments checked).
static moe_status_t lm_launch_keys(const uint16_t *h, const void *w_lm, const float *w_scale,
                                   bool w8, int32_t M, int32_t H, int32_t V, void *workspace,
                                   void *stream)
{
    unsigned long long *keys = (unsigned long long *)((char *)workspace + kWsHeader);
    const int grid = lm_grid(V);
    const int nslot = lm_lds_bytes(M, H, w8, 3) <= (size_t)kLdsDynMax ? 3 : 2;
    const size_t lds = lm_lds_bytes(M, H, w8, nslot);
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute((const void *)lmhead_kernel<false>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, kLdsDynMax);
        if (attr == hipSuccess)
            attr = hipFuncSetAttribute((const void *)lmhead_kernel<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsDynMax);
    });
    if (attr != hipSuccess)
        return MOE_ERR_LAUNCH;
    if (w8)
        hipLaunchKernelGGL(lmhead_kernel<true>, dim3(grid), dim3(kLmWaves * kWave), lds,
                           (hipStream_t)stream, (const u32x4 *)h, (const u32x4 *)w_lm, w_scale,
                           M, H, V, keys, nslot);
    else
        hipLaunchKernelGGL(lmhead_kernel<false>, dim3(grid), dim3(kLmWaves * kWave), lds,
                           (hipStream_t)stream, (const u32x4 *)h, (const u32x4 *)w_lm, nullptr,
                           M, H, V, keys, nslot);
    return check_launch();
}

// The merge phase: the keys of the GEMV's workgroups, then the verdict when
// tokens are given (arguments checked).
static moe_status_t lm_launch_merge(int32_t M, int32_t V, int32_t *argmax, float *max_logit,
                                    const int32_t *tokens, int32_t *accept,
                                    const void *workspace, void *stream)
{
    const unsigned long long *keys =
        (const unsigned long long *)((const char *)workspace + kWsHeader);
    hipLaunchKernelGGL(lmhead_merge_kernel, dim3(1), dim3(kLmWaves * kWave), 0,
                       (hipStream_t)stream, keys, lm_grid(V), M, argmax, max_logit, tokens,
                       accept);
    return check_launch();
}

// Both phases on one stream; every argument is checked before anything is
// launched.
static moe_status_t lmhead_enqueue(const uint16_t *h, const void *w_lm, const float *w_scale,
                                   bool w8, int32_t M, int32_t H, int32_t V, int32_t *argmax,
                                   float *max_logit, const int32_t *tokens,
                                   int32_t *accept, void *workspace,
                                   size_t workspace_bytes, void *stream)
{
    if (!h || !w_lm || !argmax || !workspace || (w8 && !w_scale))
        return MOE_ERR_NULL;
    if (M < 1 || H < 1 || V < 1)
        return MOE_ERR_SHAPE;
    if (M > kMaxM || H % (w8 ? 16 : 8) != 0 || H > kMaxDim ||
        lm_lds_bytes(M, H, w8) > (size_t)kLdsDynMax)
        return MOE_ERR_UNSUPPORTED;
    if (w8 && !aligned4(w_scale))
        return MOE_ERR_ALIGN;
    if (!aligned16(h) || !aligned16(w_lm) || !aligned4(argmax) ||
        (max_logit && !aligned4(max_logit)) || !aligned16(workspace) ||
        (tokens && (!aligned4(tokens) || !aligned4(accept))))
        return MOE_ERR_ALIGN;
    if (workspace_bytes < lmhead_argmax_workspace_bytes(M, V))
        return MOE_ERR_WORKSPACE;
    const moe_status_t st = lm_launch_keys(h, w_lm, w_scale, w8, M, H, V, workspace, stream);
    if (st != MOE_OK)
        return st;
    return lm_launch_merge(M, V, argmax, max_logit, tokens, accept, workspace, stream);
}

extern "C" moe_status_t lmhead_partial_keys(const uint16_t *h, const uint16_t *w_lm, int32_t M,
                                            int32_t H, int32_t V, void *workspace,
                                            size_t workspace_bytes, void *stream)
{
    const moe_status_t st =
        lm_check_keys(h, w_lm, nullptr, false, M, H, V, workspace, workspace_bytes);
    return st != MOE_OK ? st : lm_launch_keys(h, w_lm, nullptr, false, M, H, V, workspace, stream);
}

extern "C" moe_status_t lmhead_partial_keys_fp8(const uint16_t *h, const uint8_t *w_lm,
                                                const float *w_scale, int32_t M, int32_t H,
                                                int32_t V, void *workspace,
                                                size_t workspace_bytes, void *stream)
{
    const moe_status_t st =
        lm_check_keys(h, w_lm, w_scale, true, M, H, V, workspace, workspace_bytes);
    return st != MOE_OK ? st : lm_launch_keys(h, w_lm, w_scale, true, M, H, V, workspace, stream);
}

extern "C" moe_status_t lmhead_merge_keys(int32_t M, int32_t V, int32_t *argmax,
                                          float *max_logit, const int32_t *tokens,
                                          int32_t *accept, const void *workspace,
                                          size_t workspace_bytes, void *stream)
{
    const moe_status_t st =
        lm_check_merge(M, V, argmax, max_logit, tokens, accept, workspace, workspace_bytes);
    return st != MOE_OK ? st
                        : lm_launch_merge(M, V, argmax, max_logit, tokens, accept, workspace,
                                          stream);
}

extern "C" moe_status_t lmhead_argmax(const uint16_t *h, const uint16_t *w_lm,
                                      int32_t M, int32_t H, int32_t V,
                                      int32_t *argmax, float *max_logit,
                                      void *workspace, size_t workspace_bytes,
                                      void *stream)
{
    return lmhead_enqueue(h, w_lm, nullptr, false, M, H, V, argmax, max_logit, nullptr,
                          nullptr, workspace, workspace_bytes, stream);
}

extern "C" moe_status_t lmhead_argmax_fp8(const uint16_t *h, const uint8_t *w_lm,
                                          const float *w_scale, int32_t M, int32_t H,
                                          int32_t V, int32_t *argmax, float *max_logit,
                                          void *workspace, size_t workspace_bytes,
                                          void *stream)
{
    return lmhead_enqueue(h, w_lm, w_scale, true, M, H, V, argmax, max_logit, nullptr,
                          nullptr, workspace, workspace_bytes, stream);
}

extern "C" moe_status_t lmhead_greedy_verify(const uint16_t *h, const uint16_t *w_lm,
                                             const int32_t *tokens, int32_t M,
                                             int32_t H, int32_t V, int32_t *argmax,
                                             float *max_logit, int32_t *accept,
                                             void *workspace, size_t workspace_bytes,
                                             void *stream)
{
    if (!tokens || !accept)
        return MOE_ERR_NULL;
    return lmhead_enqueue(h, w_lm, nullptr, false, M, H, V, argmax, max_logit, tokens,
                          accept, workspace, workspace_bytes, stream);
}

extern "C" moe_status_t lmhead_greedy_verify_fp8(const uint16_t *h, const uint8_t *w_lm,
                                                 const float *w_scale, const int32_t *tokens,
                                                 int32_t M, int32_t H, int32_t V,
                                                 int32_t *argmax, float *max_logit,
                                                 int32_t *accept, void *workspace,
                                                 size_t workspace_bytes, void *stream)
{
    if (!tokens || !accept)
        return MOE_ERR_NULL;
    return lmhead_enqueue(h, w_lm, w_scale, true, M, H, V, argmax, max_logit, tokens,
                          accept, workspace, workspace_bytes, stream);
}
