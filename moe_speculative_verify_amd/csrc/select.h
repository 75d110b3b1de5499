// select.h -- softmax top-k selection of one token's router logits by one
// wavefront: the top-k step of the router chain of the LMSYS post "Chasing
// the batch-1 floor: Ling-3.0-flash speculative decode on Blackwell",
// section "PDL: the latency floor of stacked small kernels", Fig. 7. Used by
// the router kernel and by the up projection's prologue, which compute the
// same bits from the same logits.
#pragma once

#include "common.h"

namespace mv {

// most slices of the hidden dimension the router kernel splits a row into
constexpr int kRouteSlicesMax = 4;

// ---- per-lane sorted lists of 64-bit selection keys (order code of the
// logit << 32 | ~id: a larger key is a larger logit, or an equal logit with
// a smaller id; keys of distinct ids never tie). Written with compile-time
// indices only, so every element stays in its own registers.

template <int KJ, int A, int B, bool DESC>
__device__ __forceinline__ void sel_cex(uint64_t (&key)[KJ])
{
    const uint64_t ka = key[A], kb = key[B];
    const bool sw = DESC ? ka < kb : ka > kb;
    key[A] = sw ? kb : ka;
    key[B] = sw ? ka : kb;
}

// one bitonic stage: compare-exchange every pair (a, a ^ STRIDE)
template <int KJ, int SIZE, int STRIDE, int A>
__device__ __forceinline__ void sel_stage(uint64_t (&key)[KJ])
{
    if constexpr (A < KJ) {
        constexpr int B = A ^ STRIDE;
        if constexpr (B > A)
            sel_cex<KJ, A, B, (A & SIZE) == 0>(key);
        sel_stage<KJ, SIZE, STRIDE, A + 1>(key);
    }
}
template <int KJ, int SIZE, int STRIDE>
__device__ __forceinline__ void sel_merge(uint64_t (&key)[KJ])
{
    if constexpr (STRIDE > 0) {
        sel_stage<KJ, SIZE, STRIDE, 0>(key);
        sel_merge<KJ, SIZE, STRIDE / 2>(key);
    }
}
// bitonic sort, largest key first (KJ a power of two)
template <int KJ, int SIZE = 2>
__device__ __forceinline__ void sel_sort(uint64_t (&key)[KJ])
{
    if constexpr (SIZE <= KJ) {
        sel_merge<KJ, SIZE, SIZE / 2>(key);
        sel_sort<KJ, SIZE * 2>(key);
    }
}
// drop the head of the list where adv is set (key 0 enters at the end)
template <int KJ, int J = 0>
__device__ __forceinline__ void sel_pop(uint64_t (&key)[KJ], bool adv)
{
    if constexpr (J + 1 < KJ) {
        key[J] = adv ? key[J + 1] : key[J];
        sel_pop<KJ, J + 1>(key, adv);
    } else {
        key[J] = adv ? 0ull : key[J];
    }
}


// Selection key of logit v of expert e: order code << 32 | ~id, so a larger
// key is a larger logit or an equal logit with a smaller id (keys of
// distinct ids never tie); ids from E on get key 0, below every number
// (k <= E keeps them unselected); NaN never outranks a number; -0 and +0
// share a code.
__device__ __forceinline__ uint64_t sel_key(float v, int e, int E)
{
    uint32_t u = __float_as_uint(v != v ? -INFINITY : v);
    u = u == 0x80000000u ? 0u : u;
    const uint32_t code = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
    return e < E ? ((uint64_t)code << 32) | (uint32_t)~(uint32_t)e : 0ull;
}

// Lane s < k holds the s-th selected key (descending): its expert id and
// the softmax weight of the selected logits, taken in fp32, shifted by the
// largest, summed over the wavefront in a fixed order.
__device__ __forceinline__ void sel_softmax(uint64_t sel, int k, int lane, int &sel_idx,
                                            float &sel_w)
{
    sel_idx = (int)~(uint32_t)sel;
    const float my_v = f32_unorder((uint32_t)(sel >> 32));
    const float top = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_v), 0));
    const float ex = (lane < k) ? expf(my_v - top) : 0.0f;
    const float den = wave_sum(ex);
    sel_w = ex / den;
}

// The k largest of this wavefront's logits lv[q] (id e = lane + 64 q, ids
// from E on absent) and their softmax weights: lane s < k gets the s-th
// selection (descending logit, ties to the lower id) and its weight. Every
// lane sorts its logits by (value descending, id ascending) once; then each
// of the k rounds takes the wave-wide maximum of the lane heads (DPP on the
// 32-bit order code), breaks an equal-value tie by the lowest id, and
// advances the winning lane's list.
template <int KJ>
__device__ __forceinline__ void topk_select(const float (&lv)[KJ], int E, int k, int lane,
                                            int &sel_idx, float &sel_w)
{
    uint64_t key[KJ];
#pragma unroll
    for (int q = 0; q < KJ; ++q)
        key[q] = sel_key(lv[q], lane + kWave * q, E);
    sel_sort<KJ>(key);
    uint64_t sel = 0;                            // lane s keeps selection s
    for (int s = 0; s < k; ++s) {
        const uint64_t win = wave_max_key(key[0]);
        sel = lane == s ? win : sel;
        sel_pop<KJ>(key, key[0] == win);         // the winner's next logit moves up
    }
    sel_softmax(sel, k, lane, sel_idx, sel_w);
}

} // namespace mv
