// topk_block.hpp -- token-budget selection of one (b, head) by a whole workgroup.
//
// The rule is the one in topk_wave.hpp (SeerAttention-R, abstract: a fixed
// token budget at block granularity): k = policy count of the nc complete
// blocks; keep the k largest scores, equal scores ordered by the lower block
// id; emit the kept ids ascending, -1 after them.  Here every wave of an
// NT-thread workgroup takes part, over keys that are already in LDS:
//   * a block-wide 8-bit radix select from the top digit finds the k-th
//     largest key T and how many keys equal to T to take.  Every wave scans
//     the 256-bin histogram itself, so a pass costs one barrier; histograms
//     rotate over three buffers, and the one cleared during a pass was last
//     read two passes before.  The passes stop once the digits so far single
//     out a bin that is taken whole: every key in it is kept, so the keys
//     compare on those digits only, and the kept set is the same;
//   * one sweep in id order places each kept id: its position is the number
//     of kept ids below it, from per-wave ballot counts.
#pragma once

#include "topk_wave.hpp"

namespace seer {

template <int NT>
struct SelBlockSmem {
    static_assert(NT >= 256 && NT % 64 == 0, "one histogram bin per thread");
    static constexpr int NW = NT / 64;
    int hist[3][256];
    float red[2][NW];      // threshold policy: per-wave max and sum
    int wcnt[2][2][NW];    // per-wave counts of the id sweep, double-buffered
};

// Clears the first radix histogram.  Call it before the barrier that completes
// the keys: that barrier also orders these stores before the first pass.
template <int NT>
__device__ __forceinline__ void block_select_prepare(SelBlockSmem<NT> &sm) {
    if (threadIdx.x < 256) sm.hist[0][threadIdx.x] = 0;
}

// keys[0..nc): order_key of the complete blocks' scores, in LDS and complete.
// Selects by the policy and writes the kept ids ascending: to out[0..k) (global,
// through Mem, -1 on to k_max) when out is not null, and to kept[0..k) (LDS)
// when kept is not null.  kept may be the keys array itself: a kept id's slot
// is never above its own index, whose key every thread has read by then.
// Returns k, the same in every thread.  Every thread of the NT-thread
// workgroup calls it; the caller orders `kept` before its readers with a
// barrier.
// KR: keys per thread held in registers (ids tid + NT i, i < KR) for every pass.
template <int NT, class Mem, int KR = 8>
__device__ __forceinline__ int block_select_keys(const uint32_t *keys, int nc, const SelectPolicy &pol, int k_max,
                                                 int32_t *out, int32_t *kept, SelBlockSmem<NT> &sm) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int k = policy_count(pol, nc, k_max);
    if (pol.kind == 2 && k > 0) {  // threshold: count the blocks with probability >= tau
        float m = -INFINITY;
        for (int j = tid; j < nc; j += NT) m = fmax_fast(m, key_to_float(keys[j]));
        m = wave_max(m);
        if (lane == 0) sm.red[0][wave] = m;
        __syncthreads();
        m = sm.red[0][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) m = fmax_fast(m, sm.red[0][w]);
        float z = 0.f;
        for (int j = tid; j < nc; j += NT) z += expf(key_to_float(keys[j]) - m);
        z = wave_sum(z);
        if (lane == 0) sm.red[1][wave] = z;
        __syncthreads();
        z = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) z += sm.red[1][w];
        const float bar = pol.tau * z;
        float cnt = 0.f;
        for (int j = tid; j < nc; j += NT) cnt += expf(key_to_float(keys[j]) - m) >= bar ? 1.f : 0.f;
        cnt = wave_sum(cnt);
        __syncthreads();  // every wave has read red[0]
        if (lane == 0) sm.red[0][wave] = cnt;
        __syncthreads();
        int c = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) c += (int)sm.red[0][w];
        c = __builtin_amdgcn_readfirstlane(c);
        k = c < k ? c : k;
    }
    if (k == nc || k == 0) {  // every complete block, or none, is kept
        if (out)
            for (int i = tid; i < k_max; i += NT) Mem::sti(out + i, i < k ? i : -1);
        if (kept)
            for (int i = tid; i < k; i += NT) kept[i] = i;
        return k;
    }
    // Each thread's first KR keys (ids tid + NT i) stay in registers for every
    // pass and the sweep; keys past KR NT are read from LDS each time.
    uint32_t kreg[KR];
#pragma unroll
    for (int i = 0; i < KR; ++i) {
        const int j = tid + i * NT;
        kreg[i] = j < nc ? keys[j] : 0u;
    }
    uint32_t prefix = 0, mask = 0xFFFFFFFFu;  // the digits found so far, and the bits they cover
    int need = k;  // keys still to take among those matching `prefix` so far
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
        int *hist = sm.hist[pass % 3];
        if (tid < 256) sm.hist[(pass + 1) % 3][tid] = 0;
#pragma unroll
        for (int i = 0; i < KR; ++i)
            if (tid + i * NT < nc && (kreg[i] & hi_mask) == prefix) atomicAdd(&hist[(kreg[i] >> shift) & 255u], 1);
        for (int j = tid + KR * NT; j < nc; j += NT) {
            const uint32_t key = keys[j];
            if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
        __syncthreads();
        // lane l covers digits 255-4l .. 252-4l, in descending order
        int cnt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cnt[i] = hist[255 - 4 * lane - i];
        const int local = cnt[0] + cnt[1] + cnt[2] + cnt[3];
        const int incl = wave_inclusive_scan(local, lane);
        const int excl = incl - local;
        int digit = 0, rest = 0, whole = 0;
        {
            int cum = excl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (cum < need && cum + cnt[i] >= need) {  // the one digit where the count crosses need
                    digit = 255 - 4 * lane - i;
                    rest = need - cum;
                    whole = rest == cnt[i];
                }
                cum += cnt[i];
            }
        }
        const uint64_t hit = __ballot(excl < need && incl >= need);  // exactly one lane
        const int src = hit ? (int)__builtin_ctzll(hit) : 0;
        prefix |= (uint32_t)__builtin_amdgcn_readlane(digit, src) << shift;
        need = __builtin_amdgcn_readlane(rest, src);
        if (__builtin_amdgcn_readlane(whole, src)) {  // the bin is taken whole: no further digit matters
            mask = 0xFFFFFFFFu << shift;
            break;
        }
    }
    // Keep keys > T and the first `need` keys == T in id order (on the bits of
    // `mask`: with a bin taken whole, every key of the bin counts as equal to T
    // and `need` is its size).
    const uint32_t T = prefix;
    int gt_seen = 0, eq_seen = 0;
    for (int base = 0, round = 0, i = 0; base < nc; base += NT, round ^= 1, ++i) {
        const int j = base + tid;
        uint32_t key = 0u;
#pragma unroll
        for (int r = 0; r < KR; ++r)
            if (i == r) key = kreg[r];
        if (i >= KR) key = j < nc ? keys[j] : 0u;
        const bool gt = j < nc && (key & mask) > T, eq = j < nc && (key & mask) == T;
        const uint64_t gt_mask = __ballot(gt), eq_mask = __ballot(eq);
        if (lane == 0) {
            sm.wcnt[round][0][wave] = __popcll(gt_mask);
            sm.wcnt[round][1][wave] = __popcll(eq_mask);
        }
        __syncthreads();
        int gt_below = gt_seen + lanes_below(gt_mask), eq_below = eq_seen + lanes_below(eq_mask);
        int gt_all = gt_seen, eq_all = eq_seen;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int cg = sm.wcnt[round][0][w], ce = sm.wcnt[round][1][w];
            if (w < wave) {
                gt_below += cg;
                eq_below += ce;
            }
            gt_all += cg;
            eq_all += ce;
        }
        if (gt || (eq && eq_below < need)) {
            const int pos = gt_below + (eq_below < need ? eq_below : need);
            if (out) Mem::sti(out + pos, j);
            if (kept) kept[pos] = j;
        }
        gt_seen = gt_all;
        eq_seen = eq_all;
    }
    if (out)
        for (int i = k + tid; i < k_max; i += NT) Mem::sti(out + i, -1);
    return k;
}

}  // namespace seer
