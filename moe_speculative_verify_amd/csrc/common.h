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

// fp8 weights are OCP E4M3 codes with one fp32 scale per output row. Every
// E4M3 value is exact in bf16, so the codes are widened to bf16 in registers
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1: two codes of one 16-bit half
// per instruction, the lower byte into the lower half) and the bf16 dot
// products and MFMAs run unchanged; the row scale multiplies the fp32 sum.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// eight codes (two words) -> eight bf16 (one 16-byte chunk), in order
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(uint32_t w0, uint32_t w1)
{
    return u32x4{e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0),
                 e4m3x2_to_bf16x2<false>(w1), e4m3x2_to_bf16x2<true>(w1)};
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
// The value v of lane (lane ^ S) of the wavefront (S a power of two below
// 64; every lane active): DPP inside a quad (S = 1, 2) or a row (S = 8:
// rotate by 8), ds_swizzle inside 32 lanes (S = 4, 16: bitmask mode, xor S),
// ds_bpermute across the halves (S = 32).
template <int S>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v)
{
    const int iv = (int)v;
    if constexpr (S == 1)
        return (uint32_t)__builtin_amdgcn_update_dpp(0, iv, 0xB1, 0xF, 0xF, false);
    else if constexpr (S == 2)
        return (uint32_t)__builtin_amdgcn_update_dpp(0, iv, 0x4E, 0xF, 0xF, false);
    else if constexpr (S == 8)
        return (uint32_t)__builtin_amdgcn_update_dpp(0, iv, 0x128, 0xF, 0xF, false);
    else if constexpr (S == 4 || S == 16)
        return (uint32_t)__builtin_amdgcn_ds_swizzle(iv, 0x1F | (S << 10));
    else {
        static_assert(S == 32, "lane_xor: S in 1, 2, 4, 8, 16, 32");
        return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(((threadIdx.x & 63u) ^ 32u) << 2), iv);
    }
}

// One compare-exchange step of a bitonic sort across the wavefront: lane i
// meets lane i ^ STRIDE; in blocks of SIZE lanes that ascend ((i & SIZE) ==
// 0) the lower lane keeps the smaller key, in descending blocks the larger.
template <int SIZE, int STRIDE>
__device__ __forceinline__ uint32_t wave_sort_step(uint32_t v, int lane)
{
    const uint32_t p = lane_xor<STRIDE>(v);
    const bool up = (lane & SIZE) == 0, low = (lane & STRIDE) == 0;
    return up == low ? min(v, p) : max(v, p);
}
template <int SIZE, int STRIDE>
__device__ __forceinline__ uint32_t wave_sort_merge(uint32_t v, int lane)
{
    v = wave_sort_step<SIZE, STRIDE>(v, lane);
    if constexpr (STRIDE > 1)
        v = wave_sort_merge<SIZE, STRIDE / 2>(v, lane);
    return v;
}
// Ascending bitonic sort of one 32-bit key per lane over the 64 lanes (21
// compare-exchange steps): lane i ends with the i-th smallest key.
template <int SIZE = 2>
__device__ __forceinline__ uint32_t wave_sort_asc(uint32_t v, int lane)
{
    v = wave_sort_merge<SIZE, SIZE / 2>(v, lane);
    if constexpr (SIZE < 64)
        v = wave_sort_asc<SIZE * 2>(v, lane);
    return v;
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
__host__ __device__ inline uint32_t f32_order(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if (u == 0x80000000u)
        u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__host__ __device__ inline float f32_unorder(uint32_t u)
{
    return __builtin_bit_cast(float, (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Running first-index argmax over rows visited in ascending order: a NaN
// counts as -inf (as in the router's selection), the first row visited is
// always taken, and a later row only when strictly larger, so the result is
// the lowest row holding the maximum -- row 0 of a run whose values are all
// -inf or NaN. kNoRow marks a lane that has visited no row yet; it loses
// every tie against a real row in the cross-lane reductions.
constexpr int kNoRow = 0x7FFFFFFF;
__host__ __device__ inline void argmax_take(float &bv, int &bi, float v, int row)
{
    v = v != v ? -INFINITY : v;
    if (v > bv || bi == kNoRow) {
        bv = v;
        bi = row;
    }
}

// Merge of two running argmaxes over disjoint rows: the larger value, then
// the lower row (kNoRow, the largest int, loses every tie).
__host__ __device__ inline void argmax_merge(float &bv, int &bi, float ov, int oi)
{
    if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
    }
}
// 64-bit key of a (value, row): order code of the value above the inverted
// row, so a larger key is a larger value or an equal value at a lower row;
// and its row.
__host__ __device__ inline unsigned long long argmax_key(float v, int row)
{
    return ((unsigned long long)f32_order(v) << 32) | (uint32_t)(~(uint32_t)row);
}
__host__ __device__ inline int argmax_key_row(unsigned long long key)
{
    return (int)(~(uint32_t)key);
}

// one fused DPP step of a wave-wide uint32 maximum; rows a broadcast leaves
// out receive 0, the identity, so the move folds into v_max_u32_dpp
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint32_t max_u32_dpp(uint32_t v)
{
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWMASK, 0xF, false);
    return o > v ? o : v;
}
// maximum over the wavefront, uniform: DPP steps inside each 16-lane row,
// the rows combined with row_bcast:15 (into rows 1 and 3) and row_bcast:31
// (into rows 2 and 3), then lane 63, which has seen every lane
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max_u32_dpp<0xB1, 0xF>(v);
    v = max_u32_dpp<0x4E, 0xF>(v);
    v = max_u32_dpp<0x141, 0xF>(v);
    v = max_u32_dpp<0x140, 0xF>(v);
    v = max_u32_dpp<0x142, 0xA>(v);
    v = max_u32_dpp<0x143, 0xC>(v);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// largest 64-bit key over the wavefront, uniform: the largest high word;
// when a single lane holds it (equal logits are rare) the low word is read
// from that lane, else it is the largest low word among the lanes holding it
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v)
{
    const uint32_t hi = (uint32_t)(v >> 32);
    const uint32_t whi = wave_max_u32(hi);
    const unsigned long long at = __ballot(hi == whi);
    uint32_t wlo;
    if (__popcll(at) == 1)                       // uniform
        wlo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, __builtin_ctzll(at));
    else
        wlo = wave_max_u32(hi == whi ? (uint32_t)v : 0u);
    return ((uint64_t)whi << 32) | wlo;
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

// Every workspace layout starts with the same 4 KB header of counters, one
// per 128-byte line (device-scope atomics on one line are serialised, so
// counters that many workgroups hit sit on lines of their own), at the same
// offsets for every entry point and shape:
//   line 0         the ticket of the last-workgroup pattern
//   lines 1 .. 20  the tickets of arrival groups 1 .. 20 (arrive_last)
// Every counter is zero when a call starts and when it ends, so one
// workspace serves every entry point and shape in turn.
constexpr size_t kWsHeader = 4096;
constexpr int kWsLineWords = 32;              // words per 128-byte line
constexpr int kWsGroups = 20;                 // arrival groups the header holds

// Two-level arrival of the last-workgroup pattern, called by one thread per
// workgroup once its results are out (every thread of the workgroup has
// stored its part and passed a workgroup barrier, so those stores happen
// before this call): workgroup b counts in at the counter of group
// b / kArrivalGroup (a line of its own), the group's last arrival resets that
// counter and counts in at the ticket (word 0), and the ticket's last arrival
// gets true and resets nothing: the caller resets the ticket.
// Ordering (device / agent scope): every count is a release, so it publishes
// the results that happen before it; the last arrival of a group follows its
// count with an acquire fence, which synchronises with every release its
// count read (the counts form one read-modify-write chain), before it counts
// in at the ticket; the ticket's last arrival acquires in the same way. So
// the selecting workgroup's later loads see every workgroup's results, and
// only the two arrivals on the chain pay for an acquire (an agent-scope
// release writes back this XCD's L2, an acquire invalidates it: about 1.3 and
// 1.0 us each, measured with 256 workgroups).
// Grids of up to kArrivalGroup * kWsGroups workgroups.
constexpr int kArrivalGroup = 32;
__device__ inline bool arrive_last(unsigned *ticket)
{
    const int grp = blockIdx.x / kArrivalGroup;
    const int ng = (gridDim.x + kArrivalGroup - 1) / kArrivalGroup;
    const unsigned gsz = (unsigned)min(kArrivalGroup, (int)gridDim.x - grp * kArrivalGroup);
    unsigned *gc = ticket + kWsLineWords * (1 + grp);
    if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) != gsz - 1)
        return false;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) !=
        (unsigned)ng - 1)
        return false;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return true;
}

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
