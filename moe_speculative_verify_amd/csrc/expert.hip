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
// At verify widths (M <= 16 tokens, top-k of 512 experts) a selected expert
// serves about one (token, slot) pair, so both projections are streamed as
// matrix-vector products: the weights go straight from HBM into registers
// (128-bit non-temporal loads, 1 KB contiguous per instruction), many
// wavefronts per CU claim their blocks from an LDS counter and each waits
// for the block it issued, the tokens' vectors sit in LDS (up) or come from
// L2 with each block (down), and every lane forms eight-element dot
// products (v_dot2_f32_bf16) that fixed DPP trees sum over the wavefront. No
// floating-point atomics: results are bitwise reproducible and every pair's
// result depends only on its own token.
//
//   up       unit = (expert, row i of I): gate row and up row of the unit;
//            epilogue a = bf16(silu(g) * u) in fp32, one rounding. With fp8
//            weights an expert that serves at least kHotPairs pairs (tokens
//            that share it) is taken 8 rows at a time on the matrix cores,
//            so its codes are widened once for all of its pairs.
//   down     workgroup b owns R rows of W_down of every selected expert;
//            block sums y[pair, rows] in LDS.
//   combine  out[t, r] = sum_j w[t,j] * y[(t,j), r], slots in order, fp32,
//            at the end of the down kernel.
// Beyond the widths whose pairs' activations would fit in LDS (M*k*I*2 bytes
// beyond about 150 KB, i.e. M >= 10 at I = 1024, k = 8; a column block then
// holds several pairs) the down projection runs as the MFMA kernel below: v_mfma_f32_16x16x32_bf16 with A = 16 rows of
// W_down from a direct-to-LDS ring and B = the pairs' activations read from
// L2; its summation order differs, so batch invariance holds within each of
// the two regimes. Every workgroup rebuilds the pair grouping in LDS from
// topk_idx, which costs less than a separate launch.
//
// The shared-expert entry points (moe_expert_ffn_shared, moe_layer_shared)
// add one always-active expert per layer as one more bucket of the same
// grouping: pair M*k + t is token t's pair with it (a virtual expert id E,
// its own weight tensors, weight 1.0, added after the routed slots), so the
// same up and down launches stream it with the routed experts (the post's
// "513-expert" MoE decode, section "Two fusions and a retune").
#include "common.h"
#include "select.h"

#include <mutex>

namespace mv {

constexpr int kXKB = 512;                           // K elements per block
constexpr int kXRowPitch = kXKB * 2 + 16;           // LDS bytes per row (padded)
constexpr int kXSteps = kXKB / 32;                  // MFMA steps per block
constexpr int kXGrid = 256;                         // one workgroup per CU
constexpr int kUpPend = kWave;                      // queued up-projection outputs per wavefront
constexpr int kXLdsDynMax = 160 * 1024 - 8 * 1024;  // static LDS stays below 8 KB


// A value read from LDS that is the same in every lane, moved to a scalar
// register so that control flow and addresses built from it stay scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Expert grouping of the (token, slot) pairs, built in LDS by every
// workgroup that needs it (the grouping step of the post's MoE chain,
// section "PDL: the latency floor of stacked small kernels"): a histogram of
// the pairs over the experts (LDS atomics), one packed prefix scan over the
// experts that yields each bucket's offset, index and first column block
// at once, and a scatter of the pair ids. Buckets are ordered by expert id
// (by pair on the direct path below); the order of pairs inside a bucket is
// whatever the atomics produced, which no result depends on (every pair's
// arithmetic is its own). A bucket is cut into column blocks of at most 16
// pairs (one MFMA B operand); with distinct experts per token a bucket never
// exceeds M <= 16 pairs.
constexpr int kGroupThreads = 256;               // threads that build it (the first 256)
// With fp8 weights, column blocks of at least this many pairs run the up
// projection on the matrix cores: 8 gate and 8 up rows per unit against the
// block's pairs.
constexpr int kHotPairs = 4;
constexpr int kBinsPerThread = kMaxE / kGroupThreads;

struct Groups {
    int D;                       // distinct valid experts
    int DV;                      // column blocks
    int wsum[kGroupThreads / kWave];   // per-wavefront totals of the scan
    int bins[kMaxE];             // pairs per expert, then bucket offsets
    int16_t e[kMaxNP];           // expert of pair p, -1 if out of range
    int16_t slot[kMaxNP];        // position of pair p inside its bucket
    int16_t sorted[kMaxNP];      // pair ids, bucket by bucket
    int16_t vexp[kMaxNP];        // expert of column block v
    int16_t vbeg[kMaxNP];        // first index into sorted of block v
    int16_t vcnt[kMaxNP];        // pairs in block v (1..16)
};

// One step of an inclusive wavefront scan: add the value of lane
// (lane - shift) in the same 16-lane row (row_shr), or the last lane of the
// previous row(s) (row_bcast); lanes without a source add 0.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ int scan_step(int v)
{
    return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROWMASK, 0xF, false);
}

// Two steps, so that other prologue loads can be issued in between:
// groups_set_pairs records this thread's pair (idx = topk_idx[threadIdx.x],
// loaded by the caller) and clears the histogram, groups_finish builds the
// buckets (it starts with a barrier). The first kGroupThreads threads do the
// work; further whole wavefronts (workgroups of 512) only join the barriers.
__device__ inline void groups_set_pairs(int idx, int NP, int E, Groups &g)
{
    const int p = threadIdx.x;
    if (p >= kGroupThreads)
        return;
    if (p < NP)
        g.e[p] = (int16_t)((idx >= 0 && idx < E) ? idx : -1);
#pragma unroll
    for (int i = 0; i < kBinsPerThread; ++i)
        g.bins[i * kGroupThreads + p] = 0;
}

// At most 64 pairs (M <= 8 at k = 8): wavefront 0 builds the buckets alone,
// behind one barrier. With at most 16 pairs whose valid experts are all
// distinct (one verify token: the router never picks an expert twice for a
// token) every valid pair is a bucket and a column block of its own, in
// pair order, read off the ids with readlane compares and a ballot.
// Otherwise the pairs' (expert, pair) keys are sorted across the wavefront
// (bitonic), the lanes where the expert changes start the buckets, and each
// bucket is cut into column blocks of 16 from its first lane. Either way the
// blocks hold what the histogram would build, in another order, which no
// result depends on. Above 64 pairs the histogram below runs.
// first_e (the shared expert, or -1): its blocks come first, the others
// keep expert order. Its bucket holds every token, so its blocks cost the
// most arithmetic; taken last they would leave a tail of it after the
// streaming has ended. nhot (LDS, zero on entry, or null): incremented by the
// number of column blocks of at least kHotPairs pairs.
constexpr int kDirectNP = 16;

__device__ inline void groups_finish(int NP, Groups &g, int first_e = -1, int *nhot = nullptr)
{
    const int p = threadIdx.x;
    const int lane = p & (kWave - 1), wave = p / kWave;
    const bool gp = p < kGroupThreads;           // uniform per wavefront
    lds_barrier();
    if (NP <= kWave) {                           // uniform
        if (wave == 0) {
            const int ep = p < NP ? g.e[p] : -1;
            bool dup = NP > kDirectNP;
            for (int q = 0; q < NP && NP <= kDirectNP; ++q) {
                const int eq = __builtin_amdgcn_readlane(ep, q);
                dup = dup || (q < p && ep >= 0 && eq == ep);
            }
            if (__ballot(dup) == 0) {
                const unsigned long long val = __ballot(ep >= 0);
                // valid pairs before this one: its block index
                const int v = __builtin_amdgcn_mbcnt_hi(
                    (uint32_t)(val >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)val, 0u));
                if (ep >= 0) {
                    g.vexp[v] = (int16_t)ep;
                    g.vbeg[v] = (int16_t)v;
                    g.vcnt[v] = 1;
                    g.sorted[v] = (int16_t)p;
                }
                if (lane == 0) {
                    g.D = __popcll(val);
                    g.DV = __popcll(val);
                }
            } else {
                // key (expert + 1, or 0 for first_e) << 8 | pair, invalid
                // pairs (and lanes past NP) last
                const uint32_t eord = ep == first_e ? 0u : (uint32_t)ep + 1u;
                uint32_t key = ep >= 0 ? (eord << 8) | (uint32_t)p : 0xFFFFFFFFu;
                key = wave_sort_asc(key, lane);
                const bool valid = key != 0xFFFFFFFFu;
                const int e = (key >> 8) == 0 ? first_e : (int)(key >> 8) - 1;
                const int pr = (int)(key & 0xFFu);
                const int nvalid = __popcll(__ballot(valid));      // lanes 0 .. nvalid - 1
                const int eprev = __builtin_amdgcn_ds_bpermute((int)(((unsigned)lane + 63u) & 63u) << 2, e);
                const bool bstart = valid && (lane == 0 || e != eprev);
                const unsigned long long smask = __ballot(bstart);
                const unsigned long long upto = (2ull << lane) - 1ull;     // lanes 0 .. lane
                const unsigned long long above = smask & ~upto;
                const int bfirst = 63 - __clzll(smask & upto);   // this bucket's first lane
                const int bend = above ? __ffsll(above) - 1 : nvalid;
                const bool vstart = valid && (lane - bfirst) % 16 == 0;
                const unsigned long long cmask = __ballot(vstart);
                const int v = __popcll(cmask & upto) - 1;
                if (valid)
                    g.sorted[lane] = (int16_t)pr;
                if (vstart) {
                    g.vexp[v] = (int16_t)e;
                    g.vbeg[v] = (int16_t)lane;
                    g.vcnt[v] = (int16_t)min(16, bend - lane);
                }
                const int nh = __popcll(__ballot(vstart && bend - lane >= kHotPairs));
                if (lane == 0) {
                    g.D = __popcll(smask);
                    g.DV = __popcll(cmask);
                    if (nhot)
                        *nhot = nh;
                }
            }
        }
        lds_barrier();
        return;
    }
    // histogram: each valid pair takes the next position in its bucket
    const int ep = p < NP ? g.e[p] : -1;
    if (ep >= 0)
        g.slot[p] = (int16_t)atomicAdd(&g.bins[ep], 1);
    lds_barrier();
    // packed per-expert fields, summed by one exclusive scan over experts:
    // bits 0-9 pairs (bucket offset), 10-19 non-empty buckets (bucket
    // index), 20-29 column blocks (first block); every total is <= 256
    int cnt[kBinsPerThread], pk[kBinsPerThread];
    int tsum = 0, incl = 0;
    // first_e's column blocks, which move to the front
    const int nbf = first_e >= 0 ? (g.bins[first_e] + 15) >> 4 : 0;
    if (gp) {
#pragma unroll
        for (int i = 0; i < kBinsPerThread; ++i) {
            cnt[i] = g.bins[p * kBinsPerThread + i];
            pk[i] = cnt[i] | ((cnt[i] > 0) << 10) | (((cnt[i] + 15) >> 4) << 20);
            tsum += pk[i];
        }
        incl = tsum;
        incl = scan_step<0x111, 0xF>(incl);          // row_shr:1
        incl = scan_step<0x112, 0xF>(incl);          // row_shr:2
        incl = scan_step<0x114, 0xF>(incl);          // row_shr:4
        incl = scan_step<0x118, 0xF>(incl);          // row_shr:8
        incl = scan_step<0x142, 0xA>(incl);          // row_bcast:15
        incl = scan_step<0x143, 0xC>(incl);          // row_bcast:31
        if (lane == kWave - 1)
            g.wsum[wave] = incl;
    }
    lds_barrier();
    if (gp) {
        int run = incl - tsum;
        for (int w = 0; w < wave; ++w)
            run += g.wsum[w];
        if (p == kGroupThreads - 1) {
            const int tot = run + tsum;
            g.D = (tot >> 10) & 1023;
            g.DV = tot >> 20;
        }
#pragma unroll
        for (int i = 0; i < kBinsPerThread; ++i) {
            const int off = run & 1023, v0 = run >> 20;
            const int expert = p * kBinsPerThread + i;
            g.bins[expert] = off;                     // bucket offset for the scatter
            for (int o = 0; o < cnt[i]; o += 16) {
                const int v = expert == first_e ? o / 16
                                                : v0 + o / 16 + (expert < first_e ? nbf : 0);
                g.vexp[v] = (int16_t)expert;
                g.vbeg[v] = (int16_t)(off + o);
                g.vcnt[v] = (int16_t)(cnt[i] - o < 16 ? cnt[i] - o : 16);
            }
            run += pk[i];
        }
        if (nhot) {
            int nh = 0;                                  // this thread's hot blocks
#pragma unroll
            for (int i = 0; i < kBinsPerThread; ++i)
                nh += cnt[i] / 16 + (cnt[i] % 16 >= kHotPairs ? 1 : 0);
            if (nh)
                atomicAdd(nhot, nh);
        }
    }
    lds_barrier();
    if (ep >= 0)
        g.sorted[g.bins[ep] + g.slot[p]] = (int16_t)p;
    lds_barrier();
}

__device__ inline void build_groups(const int *__restrict__ topk_idx, int NP, int E, Groups &g)
{
    const int idx = (int)threadIdx.x < NP ? topk_idx[threadIdx.x] : -1;
    groups_set_pairs(idx, NP, E, g);
    groups_finish(NP, g);
}

static_assert(sizeof(Groups) + 64 <= 8 * 1024, "static LDS margin");
// (every expert kernel's workgroups have at least kGroupThreads threads:
// checked where their sizes are set)

// Pairs: p < NP = M*k are routed (token p / k, slot p % k); with a shared
// expert (ns = 1) p = NP + t is token t's pair with it, expert id E.
__device__ __forceinline__ int pair_token(int p, int NP, int k)
{
    return p < NP ? p / k : p - NP;
}
__device__ __forceinline__ int pair_expert(const int *__restrict__ topk_idx, int p, int NP,
                                           int NPT, int E)
{
    return p < NP ? topk_idx[p] : (p < NPT ? E : -1);
}


// ----------------------------------------------------------------- down
// Workgroup b owns R output rows r0 .. r0+R-1 for every expert; its WV
// wavefronts claim the column blocks one at a time from an LDS counter and
// stream the R rows of W_down[e] of each (1 KB per row per K block) through
// an NB-slot direct-to-LDS ring. The B fragments (the pairs' activations,
// L2-resident) are loaded at the start of their block, ahead of the next
// weight block. Per-pair results y land in LDS and the workgroup finishes
// with the weighted combine over slots in order, so no other kernel and no
// cross-workgroup traffic is needed.
template <int R, int NB, int WV>
__global__ __launch_bounds__(WV * kWave) void expert_down_kernel(
    const u32x4 *__restrict__ act, const int *__restrict__ topk_idx,
    const float *__restrict__ topk_w, const u32x4 *__restrict__ wd,
    const u32x4 *__restrict__ wds, int M, int H, int I, int E, int k, int ns,
    float *__restrict__ out)
{
    constexpr int kBlk = R * kXRowPitch;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ Groups g;
    __shared__ int s_next;                               // the workgroup's next column block
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int nch = I / 8;                               // K = I here
    const int nkb = (I + kXKB - 1) / kXKB;
    const int r0 = blockIdx.x * R;
    const int nr = min(R, H - r0);
    unsigned char *ring = smem + wave * NB * kBlk;
    float *y_s = (float *)(smem + WV * NB * kBlk);       // [NPT][R]
    const int NP = M * k, NPT = NP + ns * M;
    float *s_tw = y_s + NPT * R;                         // [NP] routing weights

    {
        const int id = pair_expert(topk_idx, threadIdx.x, NP, NPT, E);
        const float pw = (int)threadIdx.x < NP ? topk_w[threadIdx.x] : 0.0f;
        groups_set_pairs(id, NPT, E + ns, g);
        if ((int)threadIdx.x < NP)
            s_tw[threadIdx.x] = pw;
        if (threadIdx.x == 0)
            s_next = 0;
        groups_finish(NPT, g, ns ? E : -1);              // (its barriers also publish s_next)
    }

    const int DV = uniform(g.DV);
    const int j = lane & 15, gq = lane >> 4;
    const bool row_ok = j < nr;
    // Tag of a block: column block v * 16 + K block kb, or -1 past the end;
    // a column block's K blocks stay on the wavefront that claimed it
    auto claim = [&]() {                                 // uniform: a column block, or -1
        int c = 0;
        if (lane == 0)
            c = __hip_atomic_fetch_add(&s_next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        c = uniform(__builtin_amdgcn_readlane(c, 0));
        return c < DV ? c : -1;
    };
    int cur_v = claim(), cur_kb = 0;                     // the next block to issue
    auto next_tag = [&]() {
        int t = -1;
        if (cur_v >= 0) {
            t = cur_v * 16 + cur_kb;
            if (++cur_kb == nkb) {
                cur_kb = 0;
                cur_v = claim();
            }
        }
        return t;
    };

    // Block of a tag: R rows of W_down[e], 1 KB per row, into a ring slot. A
    // -1 tag loads a cached dummy (act, clamped) with the same number of
    // loads, so every wait is one constant count.
    const u32x4 *dummy = act + min(lane, NPT * nch - 1);
    auto issue = [&](int tag, unsigned char *slot) {
        const bool real = tag >= 0;
        const int v = real ? tag >> 4 : 0, kb = real ? tag & 15 : 0;
        const int ev = uniform(g.vexp[min(v, kMaxNP - 1)]);
        const u32x4 *base = ev >= E ? wds : wd + (size_t)ev * H * nch;
        int c = kb * (kXKB / 8) + lane;
        c = c < nch ? c : nch - 1;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = min(r0 + r, H - 1);          // rows past H: unused
            load_lds16(real ? base + (size_t)row * nch + c : dummy, slot + r * kXRowPitch);
        }
    };

    // tg[q]: the tag of ring slot q. With NB > 1 the block NB - 1 ahead is
    // issued before the current one is consumed; with NB = 1 each block is
    // issued right behind its B fragments and waited for at once.
    int tg[NB];
#pragma unroll
    for (int q = 0; q < NB - 1; ++q) {
        tg[q] = next_tag();
        issue(tg[q], ring + q * kBlk);
    }
    if constexpr (NB == 1)
        tg[0] = next_tag();
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (bool live = true; live;) {
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            if (tg[q] < 0) {                             // uniform: nothing left
                live = false;
                break;
            }
            const int v = tg[q] >> 4, kb = tg[q] & 15;
            const int npair = uniform(g.vcnt[v]);
            const bool col_ok = j < npair;
            // B fragments of this block (pair j's activation chunks for K
            // group gq, L2-resident), issued before the next weight block so
            // that one wait covers both them and this block's weights (loads
            // retire in order)
            const int p = g.sorted[uniform(g.vbeg[v]) + (col_ok ? j : 0)];
            u32x4 bf[kXSteps];
#pragma unroll
            for (int s = 0; s < kXSteps; ++s) {              // (no load where no pair)
                const int c = min(kb * (kXKB / 8) + 4 * s + gq, nch - 1);
                bf[s] = col_ok ? act[(size_t)p * nch + c] : u32x4{0, 0, 0, 0};
            }
            const int nq = (q + NB - 1) % NB;
            if constexpr (NB > 1) {
                tg[nq] = next_tag();
                issue(tg[nq], ring + nq * kBlk);
            } else {
                issue(tg[0], ring);
            }
            // this block's B loads and weights (and everything older) have
            // landed; the newest weight block stays in flight
            wait_vmcnt<(NB - 1) * R>();
            const unsigned char *slot = ring + q * kBlk + (row_ok ? j : 0) * kXRowPitch + gq * 16;
#pragma unroll
            for (int s = 0; s < kXSteps; ++s) {
                u32x4 a = *(const MV_LDS u32x4 *)(slot + s * 64);
                if (!row_ok)
                    a = u32x4{0, 0, 0, 0};
                u32x4 bv = bf[s];
                if (!col_ok || kb * (kXKB / 8) + 4 * s + gq >= nch)
                    bv = u32x4{0, 0, 0, 0};
                acc = mfma_bf16(a, bv, acc);
            }
            if (kb == nkb - 1) {
                if (col_ok) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (4 * gq + r < nr)
                            y_s[p * R + 4 * gq + r] = acc[r];
                }
                acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
            if constexpr (NB == 1)
                tg[0] = next_tag();
        }
    }
    wait_vmcnt<0>();                                     // dummy loads have landed
    __syncthreads();

    // weighted combine, slots in order, fp32 (eight slots' values read at a
    // time)
    for (int i = threadIdx.x; i < M * nr; i += blockDim.x) {
        const int t = i / nr, rr = i % nr;
        float sum = 0.0f;
        for (int j0 = 0; j0 < k; j0 += 8) {
            float tw[8], y[8];
            int e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int p = t * k + min(j0 + q, k - 1);
                e[q] = j0 + q < k ? g.e[p] : -1;
                tw[q] = s_tw[p];
                y[q] = y_s[p * R + rr];
            }
#pragma unroll
            for (int q = 0; q < 8; ++q)
                sum = e[q] >= 0 ? fmaf(tw[q], y[q], sum) : sum;
        }
        if (ns)                                          // the shared expert, weight 1
            sum += y_s[(NP + t) * R + rr];
        out[(size_t)t * H + r0 + rr] = sum;
    }
}

// ---------------------------------------------------------------- GEMVs
// At verify widths a selected expert serves about one (token, slot) pair, so
// both projections are streamed as matrix-vector products: the weights go
// straight from HBM into registers (1 KB contiguous per load instruction:
// lane i takes 16-byte chunk i), each wavefront waits for the block it
// issued before it consumes it while the CU's other wavefronts keep the
// loads flowing, and every lane forms eight-element dot products
// (v_dot2_f32_bf16) that fixed DPP trees sum over the wavefront.

constexpr int kDnKB = 512;                       // down: K elements per block (bf16)
constexpr int kDnCh = kDnKB / 8;                 // 16-byte chunks per row per block

// Sum over the wavefront in a fixed order, returned uniform: the 16-lane row
// butterfly, then row 1 += row 0 and row 3 += row 2 (row_bcast:15), then
// row 3 += row 1 (row_bcast:31); lane 63 holds (r3 + r2) + (r1 + r0).
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float add_dpp_step(float v)
{
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                   0, __builtin_bit_cast(int, v), CTRL, ROWMASK, 0xF, false));
}
__device__ __forceinline__ float wave_total(float v)
{
    v = add_dpp_step<0xB1, 0xF>(v);
    v = add_dpp_step<0x4E, 0xF>(v);
    v = add_dpp_step<0x141, 0xF>(v);
    v = add_dpp_step<0x140, 0xF>(v);
    v = add_dpp_step<0x142, 0xA>(v);
    v = add_dpp_step<0x143, 0xC>(v);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// ------------------------------------------------------------ up (GEMV)
// Units are (column block v, row i of I), in order, so the chip streams one
// moving window of the weights; a block is the unit's gate row and up row,
// KC loads of 1 KB each per matrix per K block, streamed into registers.
// The units are dealt to the workgroups (one per CU) in rounds (up_count,
// up_unit below), and a workgroup's kUpWaves wavefronts claim its units one
// at a time from an LDS counter, each waiting for the block it just issued:
// a SIMD serves its older wavefront first, and the claims let that one take
// more units instead of the younger ones ending last. For every pair of the
// column block each lane forms its gate and up partial dots and two DPP
// trees reduce them; lane 0 queues the sums, and every 64 queued outputs the
// 64 lanes take a = bf16(silu(g) * u) (fp32, one rounding), one output each.
// With more than KC * 64 chunks per row a unit spans several K blocks, whose
// sums are added in LDS in block order. With fp8 weights the column blocks
// of at least kHotPairs pairs are taken first, 8 rows per unit on the matrix
// cores (below).
constexpr int kUpWaves = 12;                     // wavefronts per workgroup

// LDS row of x, in 16-byte chunks: the unit's K blocks
__host__ __device__ inline int up_x_pitch(int H, int KC, bool w8)
{
    const int nwc = w8 ? H / 16 : H / 8;
    const int nbu = (nwc + KC * kWave - 1) / (KC * kWave);
    return nbu * KC * kWave * (w8 ? 2 : 1);
}
__host__ __device__ inline size_t up_x_bytes(int M, int H, int KC, bool w8, bool xr)
{
    if (xr)
        return 0;
    return align_up((size_t)M * up_x_pitch(H, KC, w8) * 16, 256);
}
// x of the M tokens in whole K blocks (none when x sits in registers), then
// each streaming wavefront's queue of finished sums and its 16 running sums
__host__ __device__ inline size_t up_lds_bytes(int M, int H, int KC, bool w8, bool xr)
{
    return up_x_bytes(M, H, KC, w8, xr) +
           (size_t)kUpWaves * (kUpPend * (sizeof(float2) + 4) + 16 * sizeof(float2));
}

// Row of unit u (column block u / I): rotated by the block index, so the
// rows a workgroup (and so an XCD: workgroup b runs on XCD b % 8) streams
// change residue from one column block to the next. Paired A/B of the layer
// (both builds in one process, calls alternated on cold layers, 96-160
// pairs): 0.2-1.0 us less per call at M = 6, 0.3-0.5 at M = 1,
// 0.8 at M = 16. (In-kernel timestamps show the up kernel's workgroups on
// odd XCDs ending 5-12 us after those on even XCDs, with or without the
// rotation; the down kernels show no such split.)
__host__ __device__ inline int up_row(int u, int I)
{
    return (u % I + u / I) % I;
}

// The units of workgroup b. Workgroup b runs on XCD b % 8 (workgroups are
// dealt to the XCDs in turn), and under a full-chip read the odd-numbered
// XCDs stream several percent slower than the even ones (a plain streaming
// probe with no arithmetic shows it for every row pattern, as do the up
// kernel's per-XCD end times). So the units come in periods of R rounds of G
// (one unit per workgroup, dealt in turn: a moving window, every column block
// spread over every workgroup) plus one unit for each even-numbered
// workgroup: those take R + 1 units per period, the odd ones R. A partial
// last period deals its rounds first. R = 0: plain rounds. Every unit is
// taken exactly once whatever the placement; only the balance depends on it.
// Paired A/B of the layer (both builds in one process, calls alternated on
// cold layers): bf16 with R = 10, 1.4 us less at M = 6 and 3.5 us less at
// M = 16, no change at M = 1 and on Zipf-routed M = 16; the fp8 kernel, which
// streams below the chip's read rate, got slower with any R (10, 20, 30), so
// it keeps plain rounds.
__host__ __device__ inline int up_count(int N, int b, int G, int R)
{
    if (R == 0)
        return N > b ? (N - 1 - b) / G + 1 : 0;
    const int ge = (G + 1) / 2, P = R * G + ge;          // units per period
    const int F = N / P, rem = N - F * P;
    const bool even = (b & 1) == 0;
    const int ord = min(rem, R * G);                     // the partial period's rounds
    int n = F * (R + (even ? 1 : 0)) + (ord > b ? (ord - 1 - b) / G + 1 : 0);
    if (even && rem - R * G > b / 2)
        ++n;
    return n;
}
__host__ __device__ inline int up_unit(int j, int N, int b, int G, int R)
{
    if (R == 0)
        return b + G * j;
    const int ge = (G + 1) / 2, P = R * G + ge;
    const int S = R + ((b & 1) == 0 ? 1 : 0);            // slots per full period
    const int F = N / P;
    const int f = j < F * S ? j / S : F, s = j < F * S ? j % S : j - F * S;
    return f * P + (s < R ? s * G + b : R * G + b / 2);
}
constexpr int kUpRounds = 10;                    // bf16: even XCDs take 11 units to 10
constexpr int kUpRounds8 = 0;                    // fp8: plain rounds

// One wavefront, given nh = the number of column blocks of at least
// kHotPairs pairs (counted by the grouping): the block list rewritten as
// those blocks, then the others, each part in its previous order (blocks are
// independent, so no result depends on the order). The caller synchronises.
__device__ inline void hot_blocks_first(Groups &g, int lane, int nh)
{
    constexpr int kC = kMaxNP / kWave;                   // blocks per lane
    const int DV = uniform(g.DV);
    int ve[kC], vb[kC], vc[kC];
    bool ok[kC], hot[kC];
#pragma unroll
    for (int c = 0; c < kC; ++c) {
        const int v = c * kWave + lane;
        ok[c] = v < DV;
        ve[c] = ok[c] ? g.vexp[v] : 0;
        vb[c] = ok[c] ? g.vbeg[v] : 0;
        vc[c] = ok[c] ? g.vcnt[v] : 0;
        hot[c] = ok[c] && vc[c] >= kHotPairs;
    }
    int hb = 0, cb = nh;                                 // next hot / other position
#pragma unroll
    for (int c = 0; c < kC; ++c) {
        const unsigned long long mh = __ballot(hot[c]), mc = __ballot(ok[c] && !hot[c]);
        const unsigned long long m = hot[c] ? mh : mc;
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        const int pos = (hot[c] ? hb : cb) + below;
        if (ok[c]) {
            g.vexp[pos] = (int16_t)ve[c];
            g.vbeg[pos] = (int16_t)vb[c];
            g.vcnt[pos] = (int16_t)vc[c];
        }
        hb += __popcll(mh);
        cb += __popcll(mc);
    }
}

// The router's selection when it runs in the up kernel (moe_layer): the
// partial logits [nks][M][E] of the router kernel (slices of the hidden
// dimension), the optional bias, and where workgroup 0 writes the selection.
struct UpSelect {
    const float *plog;
    int nks;
    const float *bias;
    int *topk_idx;
    float *topk_w;
};
constexpr int kSelKJ = 8;                        // logits per lane: E <= 512

// KC: 16-byte chunks per lane per row and K block (a unit is one block when
// a row has at most KC * 64 chunks); W8: fp8 weights (E4M3 codes, 16 per
// chunk, an fp32 scale per row in sg / su); XR: one token and one K block
// per unit, so the lane's x chunks are the same for every unit and are
// loaded once into registers instead of staged in LDS. SEL: the expert ids
// are not given: every workgroup takes the router's softmax top-k itself from
// the partial logits (the same function and the same order as the router
// kernel, so the same bits in every workgroup), which saves the router
// kernel its cross-workgroup arrival and selection, and the expert kernels a
// reload of the ids; workgroup 0 writes the selection out.
template <int KC, bool W8, bool XR, bool SEL>
__global__ __launch_bounds__(kUpWaves * kWave) void expert_up_kernel(
    const u32x4 *__restrict__ x, const int *__restrict__ topk_idx,
    const u32x4 *__restrict__ wg, const u32x4 *__restrict__ wu,
    const u32x4 *__restrict__ wgs, const u32x4 *__restrict__ wus,
    const float *__restrict__ sg, const float *__restrict__ su, int M, int H, int I, int E,
    int k, int ns, uint16_t *__restrict__ act, UpSelect sel)
{
    constexpr int WV = kUpWaves;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ Groups g;
    __shared__ int s_next;                               // the next unit of this workgroup
    __shared__ int s_nhot;                               // hot column blocks
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int nch = H / 8;                               // 16-byte x chunks per row
    const int nwc = W8 ? H / 16 : nch;                   // 16-byte weight chunks per row
    const int nbu = (nwc + KC * kWave - 1) / (KC * kWave);   // K blocks per unit
    const int xs = up_x_pitch(H, KC, W8);                // LDS x row, chunks
    const int NP = M * k, NPT = NP + ns * M;
    const size_t xbytes = up_x_bytes(M, H, KC, W8, XR);
    u32x4 *s_x = (u32x4 *)smem;                          // [M][xs]
    // finished (gate, up) sums waiting for the SwiGLU epilogue: up to
    // kUpPend per wavefront, turned into activations 64 lanes at a time
    float2 *s_gu = (float2 *)(smem + xbytes) + wave * kUpPend;
    int *s_ai = (int *)((float2 *)(smem + xbytes) + WV * kUpPend) + wave * kUpPend;
    // per-pair running sums over the K blocks of a unit (up to 16 pairs)
    float2 *s_acc = (float2 *)((int *)((float2 *)(smem + xbytes) + WV * kUpPend) +
                               WV * kUpPend) + wave * 16;

    // ---- prologue: x (XR), pair ids, then the buckets
    constexpr int kXr = XR ? KC * (W8 ? 2 : 1) : 1;
    u32x4 xreg[kXr];                                     // XR: this lane's x chunks
    if constexpr (XR) {
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            const int cp = c * kWave + lane;             // the lane's weight chunk c
            if constexpr (W8) {
                const int xc = min(2 * cp, nch - 2);     // clamped; zeroed below
                xreg[2 * c] = x[xc];
                xreg[2 * c + 1] = x[xc + 1];
            } else {
                xreg[c] = x[min(cp, nch - 1)];
            }
        }
    }
    if constexpr (!XR)                                   // x into LDS while the ids are found
        stage_rows_lds(x, M, nch, s_x, xs);
    int pid;                                             // this thread's pair's expert
    if constexpr (SEL) {
        // one wavefront per token: the slices' partial sums in slice order,
        // then the bias, then the top-k and its softmax. The selection waits
        // in the epilogue queues' LDS, unused until the units start.
        int *s_sel = (int *)(smem + xbytes);
        static_assert(kUpWaves * kUpPend * sizeof(float2) >= kMaxNP * sizeof(int), "room");
        for (int t = wave; t < M; t += WV) {
            // every load unpredicated and in flight together: slices past
            // nks reread the last one (the workspace holds kRouteSlicesMax)
            // and are left out of the sum
            float pv[kRouteSlicesMax][kSelKJ], bq[kSelKJ], lv[kSelKJ];
#pragma unroll
            for (int q = 0; q < kSelKJ; ++q) {
                const int e = lane + kWave * q, ec = e < E ? e : E - 1;
#pragma unroll
                for (int sl = 0; sl < kRouteSlicesMax; ++sl)
                    pv[sl][q] = sel.plog[((size_t)min(sl, sel.nks - 1) * M + t) * E + ec];
            }
            if (sel.bias) {                              // uniform
#pragma unroll
                for (int q = 0; q < kSelKJ; ++q)
                    bq[q] = sel.bias[min(lane + kWave * q, E - 1)];
            } else {
#pragma unroll
                for (int q = 0; q < kSelKJ; ++q)
                    bq[q] = 0.0f;
            }
#pragma unroll
            for (int q = 0; q < kSelKJ; ++q) {
                float l = pv[0][q];
#pragma unroll
                for (int sl = 1; sl < kRouteSlicesMax; ++sl)
                    if (sl < sel.nks)
                        l += pv[sl][q];
                lv[q] = l + bq[q];
            }
            int si;
            float sw;
            topk_select<kSelKJ>(lv, E, k, lane, si, sw);
            if (lane < k) {
                s_sel[t * k + lane] = si;
                if (blockIdx.x == 0) {
                    sel.topk_idx[(size_t)t * k + lane] = si;
                    sel.topk_w[(size_t)t * k + lane] = sw;
                }
            }
        }
        lds_barrier();
        const int p = threadIdx.x;
        pid = p < NP ? s_sel[p] : (p < NPT ? E : -1);
    } else {
        pid = pair_expert(topk_idx, threadIdx.x, NP, NPT, E);
    }
    groups_set_pairs(pid, NPT, E + ns, g);
    if (threadIdx.x == 0) {
        s_next = 0;
        s_nhot = 0;
    }
    wait_vmcnt<0>();                                     // the pair id and x are in
    if constexpr (XR) {
#pragma unroll
        for (int c = 0; c < KC; ++c)                     // the K tail of x reads as zero
            if (c * kWave + lane >= nwc) {
#pragma unroll
                for (int i = 0; i < (W8 ? 2 : 1); ++i)
                    xreg[c * (W8 ? 2 : 1) + i] = u32x4{0, 0, 0, 0};
            }
    } else {
        for (int i = threadIdx.x; i < M * (xs - nch); i += blockDim.x) {
            const int t = i / (xs - nch), c = nch + i % (xs - nch);
            s_x[t * xs + c] = u32x4{0, 0, 0, 0};         // K padding reads as zero
        }
    }
    constexpr bool HOT = W8 && !XR;
    groups_finish(NPT, g, ns ? E : -1, HOT ? &s_nhot : nullptr);  // (its barriers also publish s_next)
    // fp8: column blocks of at least kHotPairs pairs go to the matrix cores
    // (hot units below) and move to the front: wavefront 0 rewrites the
    // block list as [hot blocks][the rest], each part in its previous order,
    // published by the barrier after x. Only an even number of them, nhot,
    // run as hot units (with I / 8 units per block every workgroup then gets
    // the same number of them); an odd one out stays first among the GEMV
    // blocks.
    if constexpr (HOT) {
        if (M >= kHotPairs && wave == 0) {               // uniform
            const int nh = uniform(s_nhot);
            if (nh >= 2)
                hot_blocks_first(g, lane, nh);
            if (lane == 0)
                s_nhot = nh & ~1;
        }
    }
    if constexpr (!XR) {
        wait_vmcnt<0>();                                 // this wave's share of x has landed
        lds_barrier();                                   // ... and every other wave's
    }
    const int nhot = HOT && M >= kHotPairs ? uniform(s_nhot) : 0;
    const int nhu = nhot * (I / 8);                      // hot units: 8 rows of a hot block
    const int nhw = up_count(nhu, (int)blockIdx.x, (int)gridDim.x, 0);   // this workgroup's
    const int nunits = (uniform(g.DV) - nhot) * I;       // GEMV units, after the hot blocks
    constexpr int kR = W8 ? kUpRounds8 : kUpRounds;
    const int nwg = up_count(nunits, (int)blockIdx.x, (int)gridDim.x, kR);

    int pend = 0;                                        // uniform
    auto flush = [&]() {
        if (lane < pend) {
            const float2 v = s_gu[lane];
            act[s_ai[lane]] = (uint16_t)f32_to_bf16_rne(v.x / (1.0f + expf(-v.x)) * v.y);
        }
        pend = 0;
    };
    // uniform: a GEMV unit (blocks from nhot on), -2 - h for hot unit h, or
    // -1 past the end. The workgroup's hot units come first.
    auto claim = [&]() {
        int j = 0;
        if (lane == 0)
            j = __hip_atomic_fetch_add(&s_next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        j = uniform(__builtin_amdgcn_readlane(j, 0));
        if constexpr (HOT) {
            if (j < nhw)
                return -2 - ((int)blockIdx.x + (int)gridDim.x * j);
            j -= nhw;
        }
        return j < nwg ? nhot * I + up_unit(j, nunits, (int)blockIdx.x, (int)gridDim.x, kR) : -1;
    };
    // Tag of a block: unit * 16 + kb, or -1 past the end; a unit's K blocks
    // stay on one wavefront. The workgroup's hot units are claimed first and
    // taken whole, below, before the first GEMV unit.
    int cur_u = claim(), cur_kb = 0;
    auto next_tag = [&]() {
        int t = -1;
        if (cur_u >= 0) {
            t = cur_u * 16 + cur_kb;
            if (++cur_kb == nbu) {
                cur_kb = 0;
                cur_u = claim();
            }
        }
        return t;
    };

    // Block of a tag: KC loads of the gate row, KC of the up row. A -1 tag
    // rereads the first kilobyte of W_gate instead, so every wait is one
    // constant.
    auto issue = [&](int tag, u32x4 (&dg)[KC], u32x4 (&du)[KC], float &sgv, float &suv) {
        const bool real = tag >= 0;
        const int u = real ? tag >> 4 : 0, kb = real ? tag & 15 : 0;
        const int v = min(u / I, kMaxNP - 1), i = up_row(u, I);
        const int ev = uniform(g.vexp[v]);
        const bool sh = real && ev >= E;                 // the shared expert's slabs
        const size_t row = real ? (size_t)(sh ? 0 : ev) * I + i : 0;   // row in its tensor
        const size_t roff = row * nwc;
        const u32x4 *bg = sh ? wgs + roff : wg + roff;   // uniform
        const u32x4 *bu = sh ? wus + roff : wu + roff;
        if constexpr (W8) {                              // the rows' scales (uniform)
            sgv = sg[row];
            suv = su[row];
        }
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            int ch = (kb * KC + c) * kWave + lane;
            ch = ch < nwc ? ch : nwc - 1;                // K tail: zeroed before use
            int off = real ? ch : min(lane, nwc - 1);
            asm volatile("" : "+v"(off));                // one load on one path: no branch
            dg[c] = load_stream(bg + off);
            du[c] = load_stream(bu + off);
        }
    };
    auto consume = [&](int tag, u32x4 (&dg)[KC], u32x4 (&du)[KC], float sgv, float suv) {
        const int u = tag >> 4, kb = tag & 15;
        const int v = u / I, i = up_row(u, I);
        const int npair = uniform(g.vcnt[v]);
        const int pb = uniform(g.vbeg[v]);
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            if ((kb * KC + c) * kWave + kWave > nwc) {   // uniform: the K tail
                const bool ok = (kb * KC + c) * kWave + lane < nwc;
                dg[c] = ok ? dg[c] : u32x4{0, 0, 0, 0};
                du[c] = ok ? du[c] : u32x4{0, 0, 0, 0};
            }
        }
        // fp8: the codes widened to bf16 once, for every pair of the unit
        constexpr int kWc = W8 ? 2 * KC : KC;            // bf16 weight chunks per lane
        u32x4 bg[kWc], bu[kWc];
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            if constexpr (W8) {
                bg[2 * c] = e4m3x8_to_bf16(dg[c].x, dg[c].y);
                bg[2 * c + 1] = e4m3x8_to_bf16(dg[c].z, dg[c].w);
                bu[2 * c] = e4m3x8_to_bf16(du[c].x, du[c].y);
                bu[2 * c + 1] = e4m3x8_to_bf16(du[c].z, du[c].w);
            } else {
                bg[c] = dg[c];
                bu[c] = du[c];
            }
        }
        // the lane's gate and up partial dots of pair p, chunks in order
        auto dots = [&](int p, float &ga, float &ua) {
            ga = 0.0f;
            ua = 0.0f;
            if constexpr (W8) {
                // chunk c holds columns 16 ch .. 16 ch + 15: x chunks 2 ch, 2 ch + 1
                const u32x4 *xr = s_x + pair_token(p, NP, k) * xs + 2 * (kb * KC * kWave + lane);
#pragma unroll
                for (int c = 0; c < KC; ++c) {
                    const u32x4 x0 = XR ? xreg[2 * c % kXr] : xr[2 * c * kWave];
                    const u32x4 x1 = XR ? xreg[(2 * c + 1) % kXr] : xr[2 * c * kWave + 1];
                    ga = dot8_bf16(bg[2 * c], x0, ga);
                    ga = dot8_bf16(bg[2 * c + 1], x1, ga);
                    ua = dot8_bf16(bu[2 * c], x0, ua);
                    ua = dot8_bf16(bu[2 * c + 1], x1, ua);
                }
            } else {
                const u32x4 *xr = s_x + pair_token(p, NP, k) * xs + kb * KC * kWave + lane;
#pragma unroll
                for (int c = 0; c < KC; ++c) {
                    const u32x4 xv = XR ? xreg[c % kXr] : xr[c * kWave];
                    ga = dot8_bf16(bg[c], xv, ga);
                    ua = dot8_bf16(bu[c], xv, ua);
                }
            }
        };
        // the unit's reduced sums of its jj-th pair: added over K blocks,
        // then queued for the epilogue
        auto finish = [&](int jj, int p, float gt, float ut) {
            if (nbu > 1) {                               // uniform
                if (kb > 0) {
                    const float2 a = s_acc[jj];
                    gt = a.x + gt;
                    ut = a.y + ut;
                }
                if (kb < nbu - 1) {
                    if (lane == 0)
                        s_acc[jj] = make_float2(gt, ut);
                    return;
                }
            }
            if constexpr (W8) {                          // the rows' scales
                gt *= sgv;
                ut *= suv;
            }
            // queued for the epilogue (lane 0 writes, the wavefront reads)
            if (lane == 0) {
                s_gu[pend] = make_float2(gt, ut);
                s_ai[pend] = p * I + i;
            }
            if (++pend == kUpPend)
                flush();
        };
        for (int jj = 0; jj < npair; ++jj) {
            const int p = uniform(g.sorted[pb + jj]);
            float ga, ua;
            dots(p, ga, ua);
            finish(jj, p, wave_total(ga), wave_total(ua));
        }
    };

    // fp8 hot unit h: rows i0 .. i0 + 7 of a hot block's gate and up
    // matrices against its (up to 16) pairs on v_mfma_f32_16x16x32_bf16.
    // A = the 16 weight rows (lane l: row l % 16, gate rows first), streamed
    // into registers one K block of 32 chunks per row at a time (each load:
    // 64 contiguous bytes of each of the 16 rows), a chunk of 16 codes widened
    // to two bf16 steps; B = the pairs' x rows from LDS (lane l: pair l % 16,
    // x chunks 2c and 2c + 1 against code chunk c). Lane l receives rows
    // 4 (l / 16) .. + 3 of pair l % 16: gate sums in lanes 0-31, up sums in
    // 32-63, each times its row's scale; lanes 0-31 take the up sums of lane
    // l + 32 and write the activations of their 4 rows. (The fp8 entry points
    // have no shared expert.)
    if constexpr (HOT) {
        while (cur_u <= -2) {                            // uniform: a hot unit, whole
            const int h = -2 - cur_u;
            const int v = h / (I / 8), i0 = 8 * (h % (I / 8));
            const int ev = uniform(g.vexp[v]);
            const int npair = uniform(g.vcnt[v]);
            const int r = lane & 15, gq = lane >> 4;
            const size_t row = (size_t)ev * I + i0 + (r & 7);
            const u32x4 *wr = (r < 8 ? wg : wu) + row * nwc;
            const bool col_ok = r < npair;
            const int p = g.sorted[uniform(g.vbeg[v]) + (col_ok ? r : 0)];
            const u32x4 *xr = s_x + pair_token(p, NP, k) * xs;
            constexpr int kHq = 8;                       // loads per lane per K block
            const int nkh = (nwc + 4 * kHq - 1) / (4 * kHq);   // K blocks of 4 kHq chunks
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int kb = 0; kb < nkh; ++kb) {
                // past the K tail the loads are clamped to the row's last
                // chunk (finite weights) and meet x's zero padding
                u32x4 a[kHq];
#pragma unroll
                for (int q = 0; q < kHq; ++q)
                    a[q] = load_stream(wr + min(kb * 4 * kHq + 4 * q + gq, nwc - 1));
                wait_vmcnt<0>();
#pragma unroll
                for (int q = 0; q < kHq; ++q) {
                    // this lane supplies row r of A and column r of B (zero
                    // past the block's pairs)
                    const int c = kb * 4 * kHq + 4 * q + gq;
                    const u32x4 a0 = e4m3x8_to_bf16(a[q].x, a[q].y);
                    const u32x4 a1 = e4m3x8_to_bf16(a[q].z, a[q].w);
                    u32x4 b0 = *(const MV_LDS u32x4 *)(xr + 2 * c);
                    u32x4 b1 = *(const MV_LDS u32x4 *)(xr + 2 * c + 1);
                    if (!col_ok) {
                        b0 = u32x4{0, 0, 0, 0};
                        b1 = u32x4{0, 0, 0, 0};
                    }
                    acc = mfma_bf16(a0, b0, acc);
                    acc = mfma_bf16(a1, b1, acc);
                }
            }
            const float *sc = (gq < 2 ? sg : su) + row - (r & 7) + 4 * (gq & 1);
#pragma unroll
            for (int j = 0; j < 4; ++j)                  // the rows' scales
                acc[j] *= sc[j];
            float upv[4];                                // lane l + 32's sums: the up rows
#pragma unroll
            for (int j = 0; j < 4; ++j)
                upv[j] = __shfl_xor(acc[j], 32);
            if (gq < 2 && col_ok) {
                uint32_t o[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float g0 = acc[2 * j], g1 = acc[2 * j + 1];
                    o[j] = f32_to_bf16_rne(g0 / (1.0f + expf(-g0)) * upv[2 * j]) |
                           (f32_to_bf16_rne(g1 / (1.0f + expf(-g1)) * upv[2 * j + 1]) << 16);
                }
                *(uint2 *)(act + (size_t)p * I + i0 + 4 * gq) = uint2{o[0], o[1]};
            }
            cur_u = claim();
        }
    }

    u32x4 wgr[KC], wur[KC];
    float sgr = 0.0f, sur = 0.0f;                        // fp8 row scales (unused for bf16)
    for (;;) {
        const int tg = next_tag();
        issue(tg, wgr, wur, sgr, sur);
        wait_vmcnt<0>();                                 // the block has landed
        if (tg < 0)                                      // uniform: nothing left
            break;
        consume(tg, wgr, wur, sgr, sur);
    }
    flush();                                             // the last queued outputs
}

// ---------------------------------------------------------- down (GEMV)
// The down projection at verify widths: with distinct experts per token a
// column block holds about one pair. The weights stream straight into
// registers -- one 1 KB load per row per K block (lane i takes 16-byte chunk
// i) -- together with the activation chunks of the column block's first
// pairs (from L2), and each wavefront waits for the block it issued before
// it consumes it; the other wavefronts of the CU keep the loads flowing.
// Per (pair, K block) every lane forms R eight-element dot products
// (v_dot2_f32_bf16) and each row is summed over the wavefront in a fixed DPP
// tree; the block sums are added over K blocks in order in the combine.
// Workgroup b owns rows r0 .. r0+R-1 of every expert; its wavefronts claim
// the (column block, K block) blocks one at a time from an LDS counter.

// K blocks of a W_down row: kDnCh 16-byte chunks, 512 bf16 or 1024 fp8
// columns
__host__ __device__ inline int down_gemv_nkb(int I, bool w8)
{
    const int nwc = w8 ? I / 16 : I / 8;
    return (nwc + kDnCh - 1) / kDnCh;
}
// LDS: the block sums [NPT][nkb][R], then the NP routing weights
__host__ __device__ inline size_t down_gemv_lds_bytes(int R, int NPT, int I, bool w8)
{
    return (size_t)NPT * (down_gemv_nkb(I, w8) * R + 1) * sizeof(float);
}
// activation chunks of the first kDnPre pairs of a column block are loaded
// together with the block's weights; further pairs are loaded when they are
// reached
constexpr int kDnPre = 2;
static_assert(kDnPre == 2, "the pair select in the GEMV down kernel takes two");

// W8: fp8 W_down (E4M3 codes, an fp32 scale per row in sd): a block is
// 1024 columns, each chunk widened to two bf16 chunks that meet two
// activation chunks; the row's scale is one more per-lane load of the block
// and multiplies the reduced sum.
template <int R, bool W8, int WV>
__global__ __launch_bounds__(WV * kWave) void expert_down_gemv_kernel(
    const u32x4 *__restrict__ act, const int *__restrict__ topk_idx,
    const float *__restrict__ topk_w, const u32x4 *__restrict__ wd,
    const u32x4 *__restrict__ wds, const float *__restrict__ sd, int M, int H, int I,
    int E, int k, int ns, float *__restrict__ out)
{
    constexpr int kAc = W8 ? 2 : 1;                      // activation chunks per lane per pair
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ Groups g;
    __shared__ int s_next;                               // the workgroup's next block to claim
    __shared__ int s_nhot;                               // (fp8) hot column blocks
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int nch = I / 8;                               // bf16 activation chunks (K = I)
    const int nwc = W8 ? I / 16 : nch;                   // weight chunks per row
    const int nkb = down_gemv_nkb(I, W8);
    const int NP = M * k, NPT = NP + ns * M;
    const int r0 = blockIdx.x * R;
    const int nr = min(R, H - r0);
    float *s_y = (float *)smem;                          // [NPT][nkb][R]
    float *s_tw = s_y + NPT * nkb * R;                   // [NP] routing weights

    // prologue: pair ids, routing weights (for the combine at the end) and
    // buckets
    const float pw = (int)threadIdx.x < NP ? topk_w[threadIdx.x] : 0.0f;
    groups_set_pairs(pair_expert(topk_idx, threadIdx.x, NP, NPT, E), NPT, E + ns, g);
    if (threadIdx.x == 0) {
        s_next = 0;
        s_nhot = 0;
    }
    wait_vmcnt<0>();                                     // only the pair id and weight are in flight
    if ((int)threadIdx.x < NP)
        s_tw[threadIdx.x] = pw;
    groups_finish(NPT, g, ns ? E : -1, W8 ? &s_nhot : nullptr);   // (its barriers also publish s_next)
    // fp8: the column blocks of at least kHotPairs pairs move to the front
    // and run on the matrix cores (below)
    int nhot = 0;                                        // uniform
    if constexpr (W8) {
        nhot = uniform(s_nhot);
        if (nhot > 0) {
            if (wave == 0)
                hot_blocks_first(g, lane, nhot);
            lds_barrier();
        }
    }

    // Blocks B = v * nkb + kb (column block v, K block kb), claimed one at a
    // time by the workgroup's wavefronts from an LDS counter (a SIMD serves
    // its older wavefront first; the claims let that one take more blocks);
    // -1 past the last.
    const int nblk = uniform(g.DV) * nkb;
    auto next_block = [&]() {                            // uniform
        int j = 0;
        if (lane == 0)
            j = __hip_atomic_fetch_add(&s_next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        j = uniform(__builtin_amdgcn_readlane(j, 0));
        return j < nblk ? j : -1;
    };
    // this lane's activation chunks of pair p in K block kb (clamped in the
    // K tail, zeroed before use)
    auto load_act = [&](int p, int kb, u32x4 (&a)[kAc]) {
        const int c = min(kAc * (kb * kDnCh + lane), nch - kAc);
#pragma unroll
        for (int i = 0; i < kAc; ++i)
            a[i] = act[(size_t)p * nch + c + i];
    };

    // fp8 hot block B (column block v < nhot, K block kb of 64 code chunks
    // per row): the R rows against the block's (up to 16) pairs on
    // v_mfma_f32_16x16x32_bf16. Lane l supplies row l % 16 of A (the row's
    // codes, widened; zero past R) and column l % 16 of B (that pair's
    // activations from L2; zero past the block's pairs and the K tail):
    // chunk c of 16 codes meets activation chunks 2c and 2c + 1. Lane l
    // receives rows 4 (l / 16) .. + 3 of pair l % 16, times each row's
    // scale, into the block sums. The workgroup's hot blocks are claimed
    // first. (The fp8 entry points have no shared expert.)
    int B = next_block();
    if constexpr (W8) {
        const int r = lane & 15, gq = lane >> 4;
        while (B >= 0 && B < nhot * nkb) {               // uniform
            const int v = B / nkb, kb = B % nkb;
            const int ev = uniform(g.vexp[v]);
            const int npair = uniform(g.vcnt[v]);
            const bool row_ok = r < nr, col_ok = r < npair;
            const u32x4 *wp = wd + ((size_t)ev * H + r0 + (row_ok ? r : 0)) * nwc;
            const int p = g.sorted[uniform(g.vbeg[v]) + (col_ok ? r : 0)];
            const u32x4 *ap = act + (size_t)p * nch;
            u32x4 a[16];
#pragma unroll
            for (int q = 0; q < 16; ++q)                 // clamped in the K tail
                a[q] = load_stream(wp + min(kb * kDnCh + 4 * q + gq, nwc - 1));
            float scl[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                scl[j] = sd[(size_t)ev * H + min(r0 + 4 * gq + j, H - 1)];
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int qr = 0; qr < 16; qr += 8) {
                u32x4 b[16];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int c = min(kb * kDnCh + 4 * (qr + q) + gq, nwc - 1);
                    b[2 * q] = ap[2 * c];
                    b[2 * q + 1] = ap[2 * c + 1];
                }
                wait_vmcnt<0>();
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const bool bok = col_ok && kb * kDnCh + 4 * (qr + q) + gq < nwc;
                    u32x4 a0 = e4m3x8_to_bf16(a[qr + q].x, a[qr + q].y);
                    u32x4 a1 = e4m3x8_to_bf16(a[qr + q].z, a[qr + q].w);
                    if (!row_ok) {
                        a0 = u32x4{0, 0, 0, 0};
                        a1 = u32x4{0, 0, 0, 0};
                    }
                    const u32x4 b0 = bok ? b[2 * q] : u32x4{0, 0, 0, 0};
                    const u32x4 b1 = bok ? b[2 * q + 1] : u32x4{0, 0, 0, 0};
                    acc = mfma_bf16(a0, b0, acc);
                    acc = mfma_bf16(a1, b1, acc);
                }
            }
            if (col_ok) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (4 * gq + j < nr)
                        s_y[(p * nkb + kb) * R + 4 * gq + j] = acc[j] * scl[j];
            }
            B = next_block();
        }
    }

    // Each block: lane i loads chunk i of the block for each of the R rows,
    // and the activation chunks of the column block's first pairs (the
    // pairs' rows sit in L2: every workgroup reads all of them), then waits
    // for all of it and consumes the block.
    for (;; B = next_block()) {
        if (B < 0)                                       // uniform
            break;
        const int v = B / nkb, kb = B % nkb;
        const int npair = uniform(g.vcnt[v]);
        const int pb = uniform(g.vbeg[v]);
        const int ev = uniform(g.vexp[v]);
        const bool sh = ev >= E;                         // the shared expert's slab
        const size_t ebase = sh ? 0 : (size_t)ev * H;    // first row of the slab
        const u32x4 *bp = sh ? wds : wd + ebase * nwc;
        int c = kb * kDnCh + lane;
        c = c < nwc ? c : nwc - 1;                       // K tail: zeroed before use
        u32x4 w[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = min(r0 + r, H - 1);          // rows past H: unused
            w[r] = load_stream(bp + (size_t)row * nwc + c);
        }
        float sdv = 1.0f;
        if constexpr (W8)                                // lane r < R: row r's scale
            sdv = sd[ebase + min(r0 + min(lane, R - 1), H - 1)];
        u32x4 ap[kDnPre][kAc];
#pragma unroll
        for (int q = 0; q < kDnPre; ++q)
            load_act(uniform(g.sorted[pb + min(q, npair - 1)]), kb, ap[q]);
        wait_vmcnt<0>();
        const bool ok = kb * kDnCh + lane < nwc;         // the K tail
        if (kb * kDnCh + kDnCh > nwc) {                  // uniform
#pragma unroll
            for (int r = 0; r < R; ++r)
                w[r] = ok ? w[r] : u32x4{0, 0, 0, 0};
        }
        for (int jj = 0; jj < npair; ++jj) {
            const int p = uniform(g.sorted[pb + jj]);
            u32x4 a[kAc];
            if (jj < kDnPre) {                           // uniform
#pragma unroll
                for (int i = 0; i < kAc; ++i)
                    a[i] = jj == 0 ? ap[0][i] : ap[kDnPre - 1][i];
            } else {
                load_act(p, kb, a);
            }
#pragma unroll
            for (int i = 0; i < kAc; ++i)
                a[i] = ok ? a[i] : u32x4{0, 0, 0, 0};
            float yv = 0.0f;
            if constexpr (W8) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float d = dot8_bf16(e4m3x8_to_bf16(w[r].x, w[r].y), a[0], 0.0f);
                    d = dot8_bf16(e4m3x8_to_bf16(w[r].z, w[r].w), a[1], d);
                    const float t = wave_total(d);
                    yv = lane == r ? t : yv;
                }
                yv *= sdv;                               // lane r: row r's scale
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float t = wave_total(dot8_bf16(w[r], a[0], 0.0f));
                    yv = lane == r ? t : yv;
                }
            }
            if (lane < nr)
                s_y[(p * nkb + kb) * R + lane] = yv;
        }
    }
    __syncthreads();

    // weighted combine, slots in order, fp32; each pair's K blocks in order
    // (eight slots' values read at a time)
    for (int i = threadIdx.x; i < M * nr; i += blockDim.x) {
        const int t = i / nr, rr = i % nr;
        float sum = 0.0f;
        for (int j0 = 0; j0 < k; j0 += 8) {
            float tw[8], y[8];
            int e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int p = t * k + min(j0 + q, k - 1);
                e[q] = j0 + q < k ? g.e[p] : -1;
                tw[q] = s_tw[p];
                y[q] = 0.0f;
            }
            for (int kb = 0; kb < nkb; ++kb) {
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    y[q] += s_y[((t * k + min(j0 + q, k - 1)) * nkb + kb) * R + rr];
            }
#pragma unroll
            for (int q = 0; q < 8; ++q)
                sum = e[q] >= 0 ? fmaf(tw[q], y[q], sum) : sum;
        }
        if (ns) {                                        // the shared expert, weight 1
            const int p = NP + t;
            float y = 0.0f;
            for (int kb = 0; kb < nkb; ++kb)
                y += s_y[(p * nkb + kb) * R + rr];
            sum += y;
        }
        out[(size_t)t * H + r0 + rr] = sum;
    }
}

// ------------------------------------------------------------------ host

// up: KC 16-byte chunks per lane per row and block (a unit is one block when
// a row has at most 5 * 64 chunks)
static int up_gemv_kc(int H, bool w8)
{
    const int need = ((w8 ? H / 16 : H / 8) + kWave - 1) / kWave;
    return need <= 5 ? need : 4;
}
// one token and one K block per unit: x in registers
static bool up_xr(int M, int H, bool w8)
{
    return M == 1 && (w8 ? H / 16 : H / 8) <= up_gemv_kc(H, w8) * kWave;
}
// rows of W_down per down workgroup: 256 workgroups at H = 2560; fp8 keeps
// 10 (16 rows of widened codes do not fit the registers of twelve
// wavefronts)
static int down_rows(int H, bool w8)
{
    return H <= 2560 || w8 ? 10 : 16;
}
// GEMV down kernel: eight claiming wavefronts per CU (twelve for fp8), each
// waiting for the block it just issued (no block ahead: more wavefronts keep
// the CU's loads flowing). Against four wavefronts one block ahead: M=6 42.6
// against 44.8 us, M=1 13.0 against 15.2, fp8 M=6 26.0 against 28.9, fp8 M=1
// 10.3 against 11.9 (three blocks ahead on four wavefronts: M=6 45.9, M=1
// 15.7).
constexpr int kDnGemvWaves = 8;
constexpr int kDnGemvWaves8 = 12;
// The GEMV down kernel serves every fp8 call and the bf16 calls whose pairs'
// activations stay below kGemvActMax bytes (M <= 9 at I = 1024, k = 8):
// there a column block holds about one pair. Wider bf16 calls take the MFMA
// kernel (several pairs per column block: a contraction).
constexpr size_t kGemvActMax = 150 * 1024;
static bool use_down_gemv(int NPT, int I, bool w8)
{
    return w8 || (size_t)NPT * I * 2 <= kGemvActMax;
}
static size_t down_lds_bytes(int R, int NB, int WV, int NPT)
{
    // the weight rings, the pairs' sums [NPT][R], the routing weights [NPT]
    return (size_t)WV * NB * R * kXRowPitch + (size_t)NPT * (R + 1) * sizeof(float);
}
// MFMA down kernel: eight claiming wavefronts, each issuing its block right
// behind the block's B fragments and waiting for both (one LDS slot each).
// Against four wavefronts with two slots: M=16 98.8 against 118.7 us, with
// Zipf-skewed routing 70.7 against 83.6 (twelve wavefronts: 98.1 and 69.5,
// but their slots do not fit at R = 16).
constexpr int kDnMfmaNB = 1;
constexpr int kDnMfmaWaves = 8;
static_assert(kUpWaves * kWave >= kGroupThreads && kDnGemvWaves * kWave >= kGroupThreads &&
                  kDnGemvWaves8 * kWave >= kGroupThreads && kDnMfmaWaves * kWave >= kGroupThreads,
              "the grouping needs a thread per histogram slice");
// Whether a call's shapes fit the LDS of the kernels that would serve it.
static bool ffn_supported(int M, int H, int I, int NPT, bool w8)
{
    const int KC = up_gemv_kc(H, w8);
    if (up_lds_bytes(M, H, KC, w8, up_xr(M, H, w8)) > (size_t)kXLdsDynMax)
        return false;
    const int R = down_rows(H, w8);
    if (use_down_gemv(NPT, I, w8))
        return down_gemv_lds_bytes(R, NPT, I, w8) <= (size_t)kXLdsDynMax;
    return down_lds_bytes(R, kDnMfmaNB, kDnMfmaWaves, NPT) <= (size_t)kXLdsDynMax;
}

// Workspace: the header, then the bf16 activations of M*(k+1) pairs (room
// for the shared-expert pairs, so one size serves both kinds of call).
static size_t ffn_ws_bytes(int32_t M, int32_t I, int32_t k)
{
    return kWsHeader + align_up((size_t)M * (k + 1) * I * sizeof(uint16_t), 256);
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
    if (I % 8 != 0 || I > kMaxDim || !ffn_supported(M, H, I, M * k, false))
        return MOE_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) ||
        !aligned16(w_down) || !aligned4(topk_idx) || !aligned4(topk_w) ||
        !aligned4(out))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

template <typename K>
static hipError_t allow_lds(K kernel)
{
    return hipFuncSetAttribute((const void *)kernel,
                               hipFuncAttributeMaxDynamicSharedMemorySize, kXLdsDynMax);
}

template <int KC>
static void up_attr(hipError_t &e)
{
    for (hipError_t r : {allow_lds(expert_up_kernel<KC, false, false, false>),
                         allow_lds(expert_up_kernel<KC, false, true, false>),
                         allow_lds(expert_up_kernel<KC, true, false, false>),
                         allow_lds(expert_up_kernel<KC, true, true, false>),
                         allow_lds(expert_up_kernel<KC, false, false, true>),
                         allow_lds(expert_up_kernel<KC, false, true, true>),
                         allow_lds(expert_up_kernel<KC, true, false, true>),
                         allow_lds(expert_up_kernel<KC, true, true, true>)})
        if (r != hipSuccess)
            e = r;
}
static hipError_t set_lds_attributes()
{
    hipError_t e = hipSuccess;
    up_attr<1>(e);
    up_attr<2>(e);
    up_attr<3>(e);
    up_attr<4>(e);
    up_attr<5>(e);
    for (hipError_t r : {allow_lds(expert_down_kernel<10, kDnMfmaNB, kDnMfmaWaves>),
                         allow_lds(expert_down_kernel<16, kDnMfmaNB, kDnMfmaWaves>),
                         allow_lds(expert_down_gemv_kernel<10, false, kDnGemvWaves>),
                         allow_lds(expert_down_gemv_kernel<16, false, kDnGemvWaves>),
                         allow_lds(expert_down_gemv_kernel<10, true, kDnGemvWaves8>)})
        if (r != hipSuccess)
            e = r;
    return e;
}

// The experts of one call: routed weights and, when ns = 1, the shared
// expert's (gate [I,H], up [I,H], down [H,I]).
// With w8 the routed tensors are fp8 codes with per-row scales sg, su, sd.
struct Experts {
    const void *wg, *wu, *wd;
    const uint16_t *wgs, *wus, *wds;
    int ns;
    bool w8;
    const float *sg, *su, *sd;
};

// Workgroups of the up kernel: one per CU, 256 on an MI355X; each asks for
// more than half of a CU's LDS, so that no CU takes two while another
// takes none.
constexpr int kUpGrid = 256;
constexpr size_t kOneWgLds = 81 * 1024;

template <int KC, bool W8, bool XR>
static void launch_up3(size_t lds, const uint16_t *x, const int *idx, const Experts &ex, int M,
                       int H, int I, int E, int k, uint16_t *act, const UpSelect *sel,
                       hipStream_t st)
{
    if (sel)
        hipLaunchKernelGGL((expert_up_kernel<KC, W8, XR, true>), dim3(kUpGrid),
                           dim3(kUpWaves * kWave), lds, st, (const u32x4 *)x, idx,
                           (const u32x4 *)ex.wg, (const u32x4 *)ex.wu, (const u32x4 *)ex.wgs,
                           (const u32x4 *)ex.wus, ex.sg, ex.su, M, H, I, E, k, ex.ns, act, *sel);
    else
        hipLaunchKernelGGL((expert_up_kernel<KC, W8, XR, false>), dim3(kUpGrid),
                           dim3(kUpWaves * kWave), lds, st, (const u32x4 *)x, idx,
                           (const u32x4 *)ex.wg, (const u32x4 *)ex.wu, (const u32x4 *)ex.wgs,
                           (const u32x4 *)ex.wus, ex.sg, ex.su, M, H, I, E, k, ex.ns, act,
                           UpSelect{});
}
template <bool W8>
static void launch_up(const uint16_t *x, const int *idx, const Experts &ex, int M, int H, int I,
                      int E, int k, uint16_t *act, const UpSelect *sel, hipStream_t st)
{
    const int KC = up_gemv_kc(H, W8);
    const bool xr = up_xr(M, H, W8);
    const size_t lds = max(up_lds_bytes(M, H, KC, W8, xr), kOneWgLds);
#define MV_UP(KC_) (xr ? launch_up3<KC_, W8, true>(lds, x, idx, ex, M, H, I, E, k, act, sel, st) \
                       : launch_up3<KC_, W8, false>(lds, x, idx, ex, M, H, I, E, k, act, sel, st))
    switch (KC) {
    case 1: MV_UP(1); break;
    case 2: MV_UP(2); break;
    case 3: MV_UP(3); break;
    case 4: MV_UP(4); break;
    default: MV_UP(5); break;
    }
#undef MV_UP
}

template <int R>
static void launch_down_gemv(const uint16_t *act, const int *idx, const float *tw,
                             const Experts &ex, int M, int H, int I, int E, int k,
                             float *out, hipStream_t st)
{
    const int grid = (H + R - 1) / R;
    const size_t lds = down_gemv_lds_bytes(R, M * k + ex.ns * M, I, ex.w8);
    if constexpr (R == 10) {
        if (ex.w8) {
            hipLaunchKernelGGL((expert_down_gemv_kernel<R, true, kDnGemvWaves8>), dim3(grid),
                               dim3(kDnGemvWaves8 * kWave), lds, st, (const u32x4 *)act, idx,
                               tw, (const u32x4 *)ex.wd, (const u32x4 *)ex.wds, ex.sd, M, H, I,
                               E, k, ex.ns, out);
            return;
        }
    }
    hipLaunchKernelGGL((expert_down_gemv_kernel<R, false, kDnGemvWaves>), dim3(grid),
                       dim3(kDnGemvWaves * kWave), lds, st, (const u32x4 *)act, idx, tw,
                       (const u32x4 *)ex.wd, (const u32x4 *)ex.wds, nullptr, M, H, I, E, k,
                       ex.ns, out);
}

template <int R>
static void launch_down_r(const uint16_t *act, const int *idx, const float *tw,
                          const Experts &ex, int M, int H, int I, int E, int k, float *out,
                          hipStream_t st)
{
    const int grid = (H + R - 1) / R;
    const size_t lds = down_lds_bytes(R, kDnMfmaNB, kDnMfmaWaves, M * k + ex.ns * M);
    hipLaunchKernelGGL((expert_down_kernel<R, kDnMfmaNB, kDnMfmaWaves>), dim3(grid),
                       dim3(kDnMfmaWaves * kWave), lds, st,
                       (const u32x4 *)act, idx, tw, (const u32x4 *)ex.wd,
                       (const u32x4 *)ex.wds, M, H, I, E, k, ex.ns, out);
}

// ws: the workspace (its header of counters at the start); data: where the
// caller's layout puts the activations
// sel: the router's selection runs in the up kernel (then topk_idx and
// topk_w are written there, by its workgroup 0, and read by the down
// kernel)
static moe_status_t ffn_enqueue(const uint16_t *x, const int32_t *topk_idx,
                                const float *topk_w, const Experts &ex,
                                int32_t M, int32_t H, int32_t I, int32_t E,
                                int32_t k, float *out, void *ws, void *data, hipStream_t st,
                                const UpSelect *sel = nullptr)
{
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] { attr = set_lds_attributes(); });
    if (attr != hipSuccess)
        return MOE_ERR_LAUNCH;
    uint16_t *act = (uint16_t *)data;
    (void)ws;
    if (ex.w8)
        launch_up<true>(x, topk_idx, ex, M, H, I, E, k, act, sel, st);
    else
        launch_up<false>(x, topk_idx, ex, M, H, I, E, k, act, sel, st);
    moe_status_t s = check_launch();
    if (s != MOE_OK)
        return s;
    const int R = down_rows(H, ex.w8);
    if (use_down_gemv(M * k + ex.ns * M, I, ex.w8)) {
        if (R == 10)
            launch_down_gemv<10>(act, topk_idx, topk_w, ex, M, H, I, E, k, out, st);
        else
            launch_down_gemv<16>(act, topk_idx, topk_w, ex, M, H, I, E, k, out, st);
    } else {
        if (R == 10)
            launch_down_r<10>(act, topk_idx, topk_w, ex, M, H, I, E, k, out, st);
        else
            launch_down_r<16>(act, topk_idx, topk_w, ex, M, H, I, E, k, out, st);
    }
    return check_launch();
}

// The shared expert's extra checks: its three tensors, 16-byte aligned,
// M*(k+1) pairs within the grouping's capacity, id E inside the histogram.
static moe_status_t shared_check(const uint16_t *wgs, const uint16_t *wus, const uint16_t *wds,
                                 int32_t M, int32_t H, int32_t I, int32_t E, int32_t k)
{
    if (!wgs || !wus || !wds)
        return MOE_ERR_NULL;
    if (M * (k + 1) > kMaxNP || E + 1 > kMaxE || I > kMaxDim ||
        !ffn_supported(M, H, I, M * (k + 1), false))
        return MOE_ERR_UNSUPPORTED;
    if (!aligned16(wgs) || !aligned16(wus) || !aligned16(wds))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

// route.hip
moe_status_t route_check(const uint16_t *x, const uint16_t *w_router,
                         const float *bias, int32_t M, int32_t H, int32_t E,
                         int32_t k, const int32_t *topk_idx, const float *topk_w,
                         const float *logits);
moe_status_t route_enqueue(const uint16_t *x, const uint16_t *w_router,
                           const float *bias, int32_t M, int32_t H, int32_t E,
                           int32_t k, int32_t *topk_idx, float *topk_w,
                           float *logits, void *ws, hipStream_t st,
                           const uint16_t *gamma, float eps, uint16_t *x_norm,
                           bool select, int *ks);

// One MoE layer step: the router, then the expert FFN on x (x_norm with the
// norm). With at most kSelKJ * 64 experts the router kernel stops at its
// partial logits and the up kernel selects (no cross-workgroup arrival, no
// reload of the ids); with more, the router kernel selects.
static moe_status_t layer_enqueue(const uint16_t *x, const uint16_t *w_router, const float *bias,
                                  const Experts &ex, int32_t M, int32_t H, int32_t I, int32_t E,
                                  int32_t k, int32_t *topk_idx, float *topk_w, float *out,
                                  void *workspace, hipStream_t st, const uint16_t *gamma = nullptr,
                                  float eps = 0.0f, uint16_t *x_norm = nullptr)
{
    const size_t r = moe_route_workspace_bytes(M, E);
    const bool fused_sel = E <= kSelKJ * kWave;
    int ks = 1;
    moe_status_t s = route_enqueue(x, w_router, bias, M, H, E, k, topk_idx, topk_w, nullptr,
                                   workspace, st, gamma, eps, x_norm, !fused_sel, &ks);
    if (s != MOE_OK)
        return s;
    const uint16_t *xe = gamma ? x_norm : x;             // the rows the experts read
    const UpSelect sel{(const float *)((const char *)workspace + kWsHeader), ks, bias, topk_idx,
                       topk_w};
    return ffn_enqueue(xe, topk_idx, topk_w, ex, M, H, I, E, k, out, workspace,
                       (char *)workspace + r, st, fused_sel ? &sel : nullptr);
}
moe_status_t norm_check(const uint16_t *gamma, float eps, const uint16_t *x_norm,
                        int32_t M, int32_t H);

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
    const Experts ex{w_gate, w_up, w_down, nullptr, nullptr, nullptr, 0, false, nullptr, nullptr, nullptr};
    return ffn_enqueue(x, topk_idx, topk_w, ex, M, H, I, E, k, out, workspace,
                       (char *)workspace + kWsHeader, (hipStream_t)stream);
}

extern "C" moe_status_t moe_expert_ffn_shared(
    const uint16_t *x, const int32_t *topk_idx, const float *topk_w, const uint16_t *w_gate,
    const uint16_t *w_up, const uint16_t *w_down, const uint16_t *w_gate_shared,
    const uint16_t *w_up_shared, const uint16_t *w_down_shared, int32_t M, int32_t H,
    int32_t I, int32_t E, int32_t k, float *out, void *workspace, size_t workspace_bytes,
    void *stream)
{
    moe_status_t s = ffn_check(x, topk_idx, topk_w, w_gate, w_up, w_down, M, H, I,
                               E, k, out);
    if (s != MOE_OK)
        return s;
    s = shared_check(w_gate_shared, w_up_shared, w_down_shared, M, H, I, E, k);
    if (s != MOE_OK)
        return s;
    if (!workspace)
        return MOE_ERR_NULL;
    if (!aligned16(workspace))
        return MOE_ERR_ALIGN;
    if (workspace_bytes < moe_expert_ffn_workspace_bytes(M, H, I, E, k))
        return MOE_ERR_WORKSPACE;
    const Experts ex{w_gate, w_up, w_down, w_gate_shared, w_up_shared, w_down_shared, 1, false,
                      nullptr, nullptr, nullptr};
    return ffn_enqueue(x, topk_idx, topk_w, ex, M, H, I, E, k, out, workspace,
                       (char *)workspace + kWsHeader, (hipStream_t)stream);
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
    // the FFN's data part starts where the route's ends; both share the
    // header at the start of the workspace
    const Experts ex{w_gate, w_up, w_down, nullptr, nullptr, nullptr, 0, false, nullptr, nullptr, nullptr};
    return layer_enqueue(x, w_router, bias, ex, M, H, I, E, k, topk_idx, topk_w, out, workspace,
                         (hipStream_t)stream);
}

// ---------------------------------------------------- moe_layer_noalloc
// The scratch of moe_layer_noalloc: one array per GPU, for the life of the
// process. In host code `scratch` only names the symbol; its device address
// (a different one on each GPU) comes from hipGetSymbolAddress and is what
// the kernels are given.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];
static_assert(kWsHeader + 4 * 16 * 1024 * 4 + 16 * 17 * 8192 * 2 <= MOE_NOALLOC_SCRATCH_BYTES,
              "the scratch holds the workspace of the largest moe_layer shape");
constexpr int kScratchDevices = 64;

// The scratch's address on the current device, looked up (and its counter
// header cleared on `st`) at the first call there; nullptr if the lookup fails.
static void *scratch_on_device(hipStream_t st)
{
    static std::mutex mu;
    static void *ptr[kScratchDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return nullptr;
        // the counters must start at zero (the kernels leave them so)
        if (moe_workspace_clear(p, kWsHeader, st) != MOE_OK)
            return nullptr;
        ptr[dev] = p;
    }
    return ptr[dev];
}

extern "C" moe_status_t moe_layer_noalloc(const uint16_t *x, const uint16_t *w_router,
                                          const float *bias, const uint16_t *w_gate,
                                          const uint16_t *w_up, const uint16_t *w_down,
                                          int32_t M, int32_t H, int32_t I, int32_t E,
                                          int32_t k, int32_t *topk_idx, float *topk_w,
                                          float *out, void *stream)
{
    moe_status_t s = route_check(x, w_router, bias, M, H, E, k, topk_idx, topk_w, nullptr);
    if (s != MOE_OK)
        return s;
    s = ffn_check(x, topk_idx, topk_w, w_gate, w_up, w_down, M, H, I, E, k, out);
    if (s != MOE_OK)
        return s;
    const size_t need = moe_layer_workspace_bytes(M, H, I, E, k);
    if (need > MOE_NOALLOC_SCRATCH_BYTES)
        return MOE_ERR_WORKSPACE;
    void *ws = scratch_on_device((hipStream_t)stream);
    if (!ws)
        return MOE_ERR_LAUNCH;
    return moe_layer(x, w_router, bias, w_gate, w_up, w_down, M, H, I, E, k, topk_idx, topk_w,
                     out, ws, need, stream);
}

extern "C" moe_status_t moe_layer_shared(
    const uint16_t *x, const uint16_t *w_router, const float *bias, const uint16_t *w_gate,
    const uint16_t *w_up, const uint16_t *w_down, const uint16_t *w_gate_shared,
    const uint16_t *w_up_shared, const uint16_t *w_down_shared, int32_t M, int32_t H,
    int32_t I, int32_t E, int32_t k, int32_t *topk_idx, float *topk_w, float *out,
    void *workspace, size_t workspace_bytes, void *stream)
{
    moe_status_t s = route_check(x, w_router, bias, M, H, E, k, topk_idx, topk_w,
                                 nullptr);
    if (s != MOE_OK)
        return s;
    s = ffn_check(x, topk_idx, topk_w, w_gate, w_up, w_down, M, H, I, E, k, out);
    if (s != MOE_OK)
        return s;
    s = shared_check(w_gate_shared, w_up_shared, w_down_shared, M, H, I, E, k);
    if (s != MOE_OK)
        return s;
    if (!workspace)
        return MOE_ERR_NULL;
    if (!aligned16(workspace))
        return MOE_ERR_ALIGN;
    if (workspace_bytes < moe_layer_workspace_bytes(M, H, I, E, k))
        return MOE_ERR_WORKSPACE;
    const Experts ex{w_gate, w_up, w_down, w_gate_shared, w_up_shared, w_down_shared, 1, false,
                      nullptr, nullptr, nullptr};
    return layer_enqueue(x, w_router, bias, ex, M, H, I, E, k, topk_idx, topk_w, out, workspace,
                         (hipStream_t)stream);
}

extern "C" moe_status_t moe_layer_rmsnorm(const uint16_t *h, const uint16_t *gamma,
                                          float eps, const uint16_t *w_router,
                                          const float *bias, const uint16_t *w_gate,
                                          const uint16_t *w_up, const uint16_t *w_down,
                                          int32_t M, int32_t H, int32_t I, int32_t E,
                                          int32_t k, uint16_t *x_norm, int32_t *topk_idx,
                                          float *topk_w, float *out, void *workspace,
                                          size_t workspace_bytes, void *stream)
{
    moe_status_t s = route_check(h, w_router, bias, M, H, E, k, topk_idx, topk_w,
                                 nullptr);
    if (s != MOE_OK)
        return s;
    s = norm_check(gamma, eps, x_norm, M, H);
    if (s != MOE_OK)
        return s;
    s = ffn_check(x_norm, topk_idx, topk_w, w_gate, w_up, w_down, M, H, I, E, k, out);
    if (s != MOE_OK)
        return s;
    if (!workspace)
        return MOE_ERR_NULL;
    if (!aligned16(workspace))
        return MOE_ERR_ALIGN;
    if (workspace_bytes < moe_layer_workspace_bytes(M, H, I, E, k))
        return MOE_ERR_WORKSPACE;
    // the route kernel writes the normalised rows; the expert kernels read
    // them after the kernel boundary
    const Experts ex{w_gate, w_up, w_down, nullptr, nullptr, nullptr, 0, false, nullptr, nullptr, nullptr};
    return layer_enqueue(h, w_router, bias, ex, M, H, I, E, k, topk_idx, topk_w, out, workspace,
                         (hipStream_t)stream, gamma, eps, x_norm);
}

// fp8 experts: E4M3 codes [E,I,H] / [E,H,I] with fp32 scales per row; H and
// I multiples of 16; the widths of the GEMV down kernel (M <= 9 at I = 1024,
// k = 8: the MFMA down kernel is bf16 only)
static moe_status_t ffn8_check(const uint16_t *x, const int32_t *topk_idx,
                               const float *topk_w, const uint8_t *w_gate, const float *s_gate,
                               const uint8_t *w_up, const float *s_up, const uint8_t *w_down,
                               const float *s_down, int32_t M, int32_t H, int32_t I,
                               int32_t E, int32_t k, const float *out)
{
    if (!x || !topk_idx || !topk_w || !w_gate || !w_up || !w_down || !s_gate || !s_up ||
        !s_down || !out)
        return MOE_ERR_NULL;
    moe_status_t s = check_moe_shape(M, H, E, k);
    if (s != MOE_OK)
        return s;
    if (I < 1)
        return MOE_ERR_SHAPE;
    if (H % 16 != 0 || I % 16 != 0 || I > kMaxDim || !ffn_supported(M, H, I, M * k, true))
        return MOE_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
        !aligned4(s_gate) || !aligned4(s_up) || !aligned4(s_down) || !aligned4(topk_idx) ||
        !aligned4(topk_w) || !aligned4(out))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

extern "C" moe_status_t moe_expert_ffn_fp8(
    const uint16_t *x, const int32_t *topk_idx, const float *topk_w, const uint8_t *w_gate,
    const float *s_gate, const uint8_t *w_up, const float *s_up, const uint8_t *w_down,
    const float *s_down, int32_t M, int32_t H, int32_t I, int32_t E, int32_t k, float *out,
    void *workspace, size_t workspace_bytes, void *stream)
{
    moe_status_t s = ffn8_check(x, topk_idx, topk_w, w_gate, s_gate, w_up, s_up, w_down,
                                s_down, M, H, I, E, k, out);
    if (s != MOE_OK)
        return s;
    if (!workspace)
        return MOE_ERR_NULL;
    if (!aligned16(workspace))
        return MOE_ERR_ALIGN;
    if (workspace_bytes < moe_expert_ffn_workspace_bytes(M, H, I, E, k))
        return MOE_ERR_WORKSPACE;
    const Experts ex{w_gate, w_up, w_down, nullptr, nullptr, nullptr, 0, true,
                     s_gate, s_up, s_down};
    return ffn_enqueue(x, topk_idx, topk_w, ex, M, H, I, E, k, out, workspace,
                       (char *)workspace + kWsHeader, (hipStream_t)stream);
}

extern "C" moe_status_t moe_layer_fp8(
    const uint16_t *x, const uint16_t *w_router, const float *bias, const uint8_t *w_gate,
    const float *s_gate, const uint8_t *w_up, const float *s_up, const uint8_t *w_down,
    const float *s_down, int32_t M, int32_t H, int32_t I, int32_t E, int32_t k,
    int32_t *topk_idx, float *topk_w, float *out, void *workspace, size_t workspace_bytes,
    void *stream)
{
    moe_status_t s = route_check(x, w_router, bias, M, H, E, k, topk_idx, topk_w, nullptr);
    if (s != MOE_OK)
        return s;
    s = ffn8_check(x, topk_idx, topk_w, w_gate, s_gate, w_up, s_up, w_down, s_down, M, H, I,
                   E, k, out);
    if (s != MOE_OK)
        return s;
    if (!workspace)
        return MOE_ERR_NULL;
    if (!aligned16(workspace))
        return MOE_ERR_ALIGN;
    if (workspace_bytes < moe_layer_workspace_bytes(M, H, I, E, k))
        return MOE_ERR_WORKSPACE;
    const Experts ex{w_gate, w_up, w_down, nullptr, nullptr, nullptr, 0, true,
                     s_gate, s_up, s_down};
    return layer_enqueue(x, w_router, bias, ex, M, H, I, E, k, topk_idx, topk_w, out, workspace,
                         (hipStream_t)stream);
}
