// common.h -- device helpers and host-side argument checks shared by the
// gfx950 kernels of the MoE verify hot path.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_verify.h"

namespace mv {

// 16-byte vector of four 32-bit words: one 128-bit global or LDS access.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define MV_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kMaxM = 16;          // verify tokens per call
constexpr int kMaxK = 16;          // experts per token
constexpr int kMaxNP = kMaxM * kMaxK;
constexpr int kMaxE = 1024;
constexpr int kMaxDim = 8192;      // largest H or I

// ------------------------------------------------------------------ device

// a.lo*b.lo + a.hi*b.hi + c on two bf16 pairs, fp32 accumulate
// (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c,
                                           false);
}

// Eight bf16 products of two 16-byte chunks added to acc.
__device__ __forceinline__ float dot8_bf16(u32x4 w, u32x4 x, float acc)
{
    acc = dot2_bf16(w.x, x.x, acc);
    acc = dot2_bf16(w.y, x.y, acc);
    acc = dot2_bf16(w.z, x.z, acc);
    acc = dot2_bf16(w.w, x.w, acc);
    return acc;
}

// Weight streams are read once per call: non-temporal 128-bit loads keep
// them from displacing the small reused tensors in the caches.
__device__ __forceinline__ u32x4 load_stream(const u32x4 *p)
{
    return __builtin_nontemporal_load(p);
}

// One DPP move: lane i receives lane ctrl(i)'s v (same-row patterns only).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <- 15-i within 16

// Sum over the 64 lanes of a wavefront; every lane gets the same total.
// DPP within each 16-lane row (every lane of a row ends with the identical
// row sum, since each step adds a commuted pair), then the four row sums in
// a fixed order. No LDS traffic; the order never depends on timing.
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    v += dpp_f32<kDppHalfMirror>(v);
    v += dpp_f32<kDppMirror>(v);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
}

// D += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate. Lane l supplies
// row (l % 16) of A and column (l % 16) of B over K elements
// [8*(l/16), 8*(l/16)+8) of the 32-element step; it receives D rows
// 4*(l/16) .. 4*(l/16)+3 of column l % 16.
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

// Direct HBM -> LDS 128-bit load (global_load_lds_dwordx4), non-temporal:
// lane i's 16 bytes land at lds_wave_base + 16*i. Completion is counted by
// vmcnt; the caller waits with wait_vmcnt before reading the LDS.
__device__ __forceinline__ void load_lds16(const void *g, void *lds_wave_base)
{
    __builtin_amdgcn_global_load_lds(g, (MV_LDS void *)lds_wave_base, 16, 0, 2);
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left alone). Direct-to-LDS loads
// have side effects and keep their program order, so a count over them is
// exact. Plain loads from read-only kernel arguments may be moved by the
// compiler (it also inserts the waits their register uses need), so with
// those in flight a nonzero count is only a scheduling hint: data that other
// wavefronts read from LDS is waited for with N = 0 unless only
// direct-to-LDS loads can follow it.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Order-preserving map of fp32 to uint32 (-0 and +0 both map to +0's code;
// larger floats give larger codes) and its inverse.
__device__ __forceinline__ uint32_t f32_order(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u)
        u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_unorder(uint32_t u)
{
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Maximum / minimum of a uint32 over the wavefront, returned uniform: DPP
// steps inside each 16-lane row, the rows combined with row broadcasts
// (row_bcast:15 into rows 1 and 3, then row_bcast:31 into rows 2 and 3), and
// lane 63, which has seen every lane, read back. Rows a broadcast leaves out
// receive the operation's identity, so they keep their own value (and the
// move folds into a DPP max/min). Branch-free.
template <int CTRL, int ROWMASK, bool MAX>
__device__ __forceinline__ uint32_t u32_dpp_step(uint32_t v)
{
    const int ident = MAX ? 0 : -1;
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(ident, (int)v, CTRL, ROWMASK, 0xF, false);
    return MAX ? (o > v ? o : v) : (o < v ? o : v);
}
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v)
{
    v = u32_dpp_step<0xB1, 0xF, MAX>(v);    // quad_perm [1,0,3,2]
    v = u32_dpp_step<0x4E, 0xF, MAX>(v);    // quad_perm [2,3,0,1]
    v = u32_dpp_step<0x141, 0xF, MAX>(v);   // row_half_mirror
    v = u32_dpp_step<0x140, 0xF, MAX>(v);   // row_mirror: row extreme everywhere
    v = u32_dpp_step<0x142, 0xA, MAX>(v);   // row_bcast:15
    v = u32_dpp_step<0x143, 0xC, MAX>(v);   // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// fp32 -> bf16 bits, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u)
        return (u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Workgroup barrier for LDS data written with ds_write/LDS atomics only:
// waits for this wavefront's LDS operations (lgkmcnt) and keeps the compiler
// from moving memory accesses across it, but leaves global loads -- and
// direct-to-LDS loads into OTHER LDS regions -- in flight. Data that arrives
// by direct-to-LDS loads needs wait_vmcnt and __syncthreads instead.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);                 // lgkmcnt(0) only
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Expert grouping of the (token, slot) pairs, built in LDS by every
// workgroup that needs it. This is the pair-axis form of the grouping the
// post describes in section "Two fusions and a retune": each pair compares
// itself with every other pair to find its rank inside its expert's bucket
// and whether it heads the bucket; nothing scales with the expert count.
// Buckets are ordered by expert id, pairs inside a bucket by pair index.
// A bucket is then cut into column blocks of at most 16 pairs (one MFMA B
// operand); with distinct experts per token a bucket never exceeds M <= 16
// pairs, so this only matters for repeated ids within a token.
struct Groups {
    int D;                       // distinct valid experts
    int DV;                      // column blocks
    int wheads[16];              // per-wavefront counts of bucket heads
    int pad_[14];
    // int16 arrays, 16-byte aligned and padded to a multiple of 8 entries
    // so that eight entries are read with one 128-bit LDS load
    alignas(16) int16_t e[kMaxNP];      // expert of pair p, -1 if out of range
    alignas(16) int16_t hd[kMaxNP];     // expert of pair p if it heads its bucket, else -1
    alignas(16) int16_t sorted[kMaxNP]; // pair ids, bucket by bucket
    alignas(16) int16_t dexp[kMaxNP];   // expert id of bucket d
    alignas(16) int16_t doff[kMaxNP];   // bucket d starts at sorted[doff[d]]
    alignas(16) int16_t dcnt[kMaxNP];   // pairs in bucket d
    alignas(16) int16_t vexp[kMaxNP];   // expert of column block v
    alignas(16) int16_t vbeg[kMaxNP];   // first index into sorted of block v
    alignas(16) int16_t vcnt[kMaxNP];   // pairs in block v (1..16)
};

// Eight consecutive int16 entries of an LDS array (index a multiple of 8).
__device__ __forceinline__ void lds_load8(const int16_t *arr, int q0, int (&v)[8])
{
    const u32x4 w = *(const u32x4 *)(arr + q0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = (int)(int16_t)(w[i] & 0xFFFFu);
        v[2 * i + 1] = (int)w[i] >> 16;
    }
}

// Every phase is parallel over pairs or buckets (the workgroup has at least
// NP <= 256 threads) and reads the shared arrays eight entries at a time,
// with no dependent LDS reads. Two steps, so that other prologue loads can
// be issued in between: groups_set_pairs records this thread's pair (idx =
// topk_idx[threadIdx.x], loaded by the caller; threads past NP pad the array
// with -1), groups_finish builds the buckets (it starts with a barrier).
__device__ inline void groups_set_pairs(int idx, int NP, int E, Groups &g)
{
    const int p = threadIdx.x;
    if (p < ((NP + 7) & ~7))
        g.e[p] = (int16_t)((p < NP && idx >= 0 && idx < E) ? idx : -1);
}

__device__ inline void groups_finish(int NP, Groups &g)
{
    const int p = threadIdx.x;
    const int NP8 = (NP + 7) & ~7;
    lds_barrier();
    // each pair against every other: its rank in (expert, pair) order, the
    // pairs below its bucket and in it, and whether it heads the bucket
    const int ep = p < NP ? g.e[p] : -1;
    int below = 0, same = 0, rank = 0, head = 0;
    if (ep >= 0) {
        head = 1;
        for (int q0 = 0; q0 < NP8; q0 += 8) {
            int eq[8];
            lds_load8(g.e, q0, eq);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int q = q0 + i;
                const bool ok = eq[i] >= 0;
                const bool lt = ok && eq[i] < ep;
                const bool eqe = ok && eq[i] == ep;
                below += lt;
                same += eqe;
                rank += lt || (eqe && q < p);
                head &= !(eqe && q < p);
            }
        }
        g.sorted[rank] = (int16_t)p;
    }
    if (p < NP8)
        g.hd[p] = (int16_t)(head ? ep : -1);
    // bucket count without atomics: a ballot per wavefront, summed after
    // the barrier
    {
        const unsigned long long hb = __ballot(head);
        if ((threadIdx.x & (kWave - 1)) == 0)
            g.wheads[threadIdx.x / kWave] = __popcll(hb);
    }
    lds_barrier();
    int D = 0;
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w)
        D += g.wheads[w];
    // bucket index of each head = heads with a smaller expert id
    if (head) {
        int d = 0;
        for (int q0 = 0; q0 < NP8; q0 += 8) {
            int hq[8];
            lds_load8(g.hd, q0, hq);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                d += hq[i] >= 0 && hq[i] < ep;
        }
        g.dexp[d] = (int16_t)ep;
        g.doff[d] = (int16_t)below;
        g.dcnt[d] = (int16_t)same;
    }
    lds_barrier();
    if (p == 0)
        g.D = D;
    // column blocks of <= 16 pairs: bucket d's blocks start after the
    // blocks of the buckets below it
    if (p < D) {
        int vstart = 0;
        for (int q0 = 0; q0 < p; q0 += 8) {
            int cq[8];
            lds_load8(g.dcnt, q0, cq);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                vstart += q0 + i < p ? (cq[i] + 15) / 16 : 0;
        }
        const int n = g.dcnt[p];
        for (int o = 0; o < n; o += 16) {
            const int v = vstart + o / 16;
            g.vexp[v] = g.dexp[p];
            g.vbeg[v] = (int16_t)(g.doff[p] + o);
            g.vcnt[v] = (int16_t)(n - o < 16 ? n - o : 16);
        }
        if (p == D - 1)
            g.DV = vstart + (n + 15) / 16;
    }
    if (p == 0 && D == 0)
        g.DV = 0;
    lds_barrier();
}

__device__ inline void build_groups(const int *__restrict__ topk_idx, int NP, int E, Groups &g)
{
    const int idx = (int)threadIdx.x < NP ? topk_idx[threadIdx.x] : -1;
    groups_set_pairs(idx, NP, E, g);
    groups_finish(NP, g);
}

// Direct-to-LDS staging of nrows rows of nch 16-byte chunks (row-major,
// contiguous) into LDS rows of pitch xs chunks: one 1 KB load per run of 64
// chunks, spread over the workgroup's wavefronts, lanes past the row end
// idle. Nothing waits here: the caller waits (vmcnt) and then synchronises.
__device__ inline void stage_rows_lds(const u32x4 *__restrict__ src, int nrows, int nch,
                                      u32x4 *dst, int xs)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwave = blockDim.x / kWave;
    const int runs = (nch + kWave - 1) / kWave;
    for (int i = wave; i < nrows * runs; i += nwave) {
        const int t = i / runs, r = i % runs;
        const int c = r * kWave + lane;
        if (c < nch)
            load_lds16(src + (size_t)t * nch + c, dst + (size_t)t * xs + r * kWave);
    }
}

// -------------------------------------------------------------------- host

// Every workspace layout starts with the same 256-byte header whose first
// word is the arrival ticket of the last-workgroup pattern; the ticket is zero
// when a call starts and when it ends, so one workspace can serve every entry
// point and shape in turn.
constexpr size_t kWsHeader = 256;

// Dynamic LDS a kernel may request: 160 KB per CU on gfx950, less a margin
// for the kernels' small static arrays.
constexpr int kLdsDynMax = 159 * 1024;

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }
__host__ __device__ inline size_t align_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

inline moe_status_t check_launch()
{
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

// Shape gates shared by the MoE entry points.
inline moe_status_t check_moe_shape(int32_t M, int32_t H, int32_t E, int32_t k)
{
    if (M < 1 || H < 1 || E < 1 || k < 1)
        return MOE_ERR_SHAPE;
    if (M > kMaxM || k > kMaxK || k > E || E > kMaxE)
        return MOE_ERR_UNSUPPORTED;
    if (H % 8 != 0 || H > kMaxDim)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

} // namespace mv
