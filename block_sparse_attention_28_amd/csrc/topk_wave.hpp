// topk_wave.hpp -- exact top-k of fp32 scores by one wavefront (device helpers).
//
// Scores become order-preserving 32-bit keys in LDS; an 8-bit-digit radix
// select (four histogram passes from the most significant digit, a DPP prefix
// sum over the 256 bins) finds the k-th largest key T and how many keys equal
// to T must be taken; a last sweep over the ids in order keeps keys > T plus
// the first `need` keys == T, placing each with a ballot + lane-mask popcount.
// The result is the k largest scores, equal scores ordered by the lower id,
// emitted in ascending id order.
#pragma once

#include "seer_device.hpp"

namespace seer {

__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (s == 0.0f) u = 0u;  // +0 and -0 compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes: DPP row shifts within 16-lane rows,
// then row broadcasts of lanes 15 and 31 into the following rows.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
    (void)lane;
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
    return v;
}

// Number of lanes below this one whose bit is set in `mask`.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Order LDS accesses of this wave (executed in issue order by the hardware).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// How many blocks a (b, head) keeps (SeerAttention v2 abstract: varying
// sparsity ratios; SeerAttention-R abstract: a token budget): kind 0 keeps
// min(k_max, nc) (the token budget, k_max = budget / block size), kind 1
// ceil(nc * num / den), kind 2 the blocks whose softmax probability over the
// row's scores is at least tau; every kind is capped by k_max and nc.
struct SelectPolicy {
    int kind, num, den;
    float tau;
};

__device__ __forceinline__ int policy_count(const SelectPolicy &p, int nc, int k_max) {
    int64_t k = nc;
    if (p.kind == 1) k = ((int64_t)nc * p.num + p.den - 1) / p.den;
    k = k < nc ? k : nc;
    k = k < k_max ? k : k_max;
    return (int)(k < 0 ? 0 : k);
}

// Inverse of order_key (both zeros come back as +0).
__device__ __forceinline__ float key_to_float(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// scores[0..n) as order-preserving keys in LDS, read through Mem.
template <class Mem>
__device__ __forceinline__ void wave_load_keys(const float *scores, int n, uint32_t *keys, int lane) {
    for (int base = 0; base < n; base += 64 * 8) {  // eight loads in flight per lane
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = base + lane + 64 * i;
            v[i] = j < n ? Mem::ldf(scores + j) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = base + lane + 64 * i;
            if (j < n) keys[j] = order_key(v[i]);
        }
    }
    wave_lds_sync();
}

// Select the k largest of the n keys in LDS (0 < k < n), write their ids
// ascending to out[0..k) through Mem.  8-bit radix passes from the top digit,
// stopping once the digits so far single out a bin that is taken whole.  hist: LDS scratch of 256 words private
// to this wave.  Every lane of the wave must call it.
template <class Mem>
__device__ __forceinline__ void wave_topk_from_keys(int n, int k, uint32_t *keys, int *hist, int32_t *out,
                                                    int lane) {
    uint32_t prefix = 0, mask = 0xFFFFFFFFu;  // the digits found so far, and the bits they cover
    int need = k;  // keys still to take among those matching `prefix` so far
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
#pragma unroll
        for (int i = 0; i < 4; ++i) hist[lane * 4 + i] = 0;
        wave_lds_sync();
        for (int j = lane; j < n; j += 64) {
            const uint32_t key = keys[j];
            if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
        wave_lds_sync();
        // lane l covers digits 255-4l .. 252-4l, in descending order
        int cnt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cnt[i] = hist[255 - 4 * lane - i];
        const int local = cnt[0] + cnt[1] + cnt[2] + cnt[3];
        const int incl = wave_inclusive_scan(local, lane);
        const int excl = incl - local;
        const uint64_t hit = __ballot(excl < need && incl >= need);
        int src = __ffsll((long long)hit) - 1;
        src = src < 0 ? 0 : src;
        int digit = 0, rest = 0, whole = 0;
        if (lane == src) {
            int cum = excl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (cum + cnt[i] >= need) {
                    digit = 255 - 4 * lane - i;
                    rest = need - cum;
                    whole = rest == cnt[i];
                    break;
                }
                cum += cnt[i];
            }
        }
        digit = __builtin_amdgcn_readlane(digit, src);
        need = __builtin_amdgcn_readlane(rest, src);
        prefix |= (uint32_t)digit << shift;
        wave_lds_sync();
        // A bin taken whole: every key in it is kept, so no further digit matters.
        if (__builtin_amdgcn_readlane(whole, src)) {
            mask = 0xFFFFFFFFu << shift;
            break;
        }
    }
    // Keep keys > T and the first `need` keys == T in id order, on the bits of `mask`.
    const uint32_t T = prefix;
    int written = 0, eq_seen = 0;
    for (int base = 0; base < n; base += 64) {
        const int j = base + lane;
        const uint32_t key = j < n ? keys[j] & mask : 0u;
        const bool eq = j < n && key == T;
        const uint64_t eq_mask = __ballot(eq);
        const bool take = j < n && (key > T || (eq && eq_seen + lanes_below(eq_mask) < need));
        const uint64_t take_mask = __ballot(take);
        const int pos = written + lanes_below(take_mask);
        if (take && pos < k) Mem::sti(out + pos, j);
        written += __popcll(take_mask);
        eq_seen += __popcll(eq_mask);
    }
}

// The k largest of scores[0..n) (0 < k < n), ids ascending, by one wave.
template <class Mem>
__device__ __forceinline__ void wave_topk_ascending(const float *scores, int n, int k, uint32_t *keys, int *hist,
                                                    int32_t *out, int lane) {
    wave_load_keys<Mem>(scores, n, keys, lane);
    wave_topk_from_keys<Mem>(n, k, keys, hist, out, lane);
}

}  // namespace seer
