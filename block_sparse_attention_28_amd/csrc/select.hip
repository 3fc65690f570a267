// select.hip -- token-budget top-k block selection.
//
// Operation ("SeerAttention-R: Sparse Attention Adaptation for Long
// Reasoning", abstract: a fixed token budget at 64/128-token block
// granularity): per (sequence, KV head) keep k = min(budget / bs, nc) complete
// blocks with the largest gate scores, equal scores ordered by the lower block
// id, and emit the kept ids in ascending order (so decoding reads memory
// forward).
//
// One wavefront per (b, head), several per workgroup, no workgroup barriers.
// Scores become order-preserving 32-bit keys held in the wave's LDS slice; an
// 8-bit-digit radix select (four histogram passes from the most significant
// digit, a wave prefix sum over the 256 bins) finds the k-th largest key T and
// how many keys equal to T must be taken.  A last sweep over the ids in order
// keeps keys > T plus the first `need` keys == T, placing each kept id with a
// ballot + lane-mask popcount, so the output is ascending by construction.
// All decisions are integer comparisons of the fp32 score bits.
#include "seer_device.hpp"
#include "seer_host.hpp"

namespace seer {

constexpr int kSelMaxBlocks = 16384 - 256;  // keys + histogram of one wave fit in 64 KiB of LDS

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

__global__ __launch_bounds__(256) void select_blocks_kernel(const float *scores, const int32_t *seqlens, int B,
                                                            int H, int nb_max, int slice, int block_size, int k_max,
                                                            int32_t *block_idx, int32_t *n_sel) {
    extern __shared__ uint32_t lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pair = blockIdx.x * (blockDim.x >> 6) + wave;  // b * H + h
    if (pair >= B * H) return;
    uint32_t *keys = lds + (size_t)wave * slice;              // [nb_max]
    int *hist = reinterpret_cast<int *>(keys + slice - 256);  // [256]

    const int b = pair / H;
    int L = seqlens[b];
    L = L < 0 ? 0 : L;
    int nc = L / block_size;
    nc = nc > nb_max ? nb_max : nc;
    const int k = k_max < nc ? k_max : nc;
    int32_t *out = block_idx + (int64_t)pair * k_max;
    if (lane == 0) n_sel[pair] = k;
    if (k == nc || k == 0) {  // every complete block, or none, is kept
        for (int i = lane; i < k_max; i += 64) out[i] = i < k ? i : -1;
        return;
    }
    const float *sc = scores + (int64_t)pair * nb_max;
    for (int base = 0; base < nc; base += 64 * 8) {  // eight loads in flight per lane
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = base + lane + 64 * i;
            v[i] = j < nc ? sc[j] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = base + lane + 64 * i;
            if (j < nc) keys[j] = order_key(v[i]);
        }
    }

    uint32_t prefix = 0;
    int need = k;  // keys still to take among those matching `prefix` so far
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
#pragma unroll
        for (int i = 0; i < 4; ++i) hist[lane * 4 + i] = 0;
        wave_lds_sync();
        for (int j = lane; j < nc; j += 64) {
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
        int digit = 0, rest = 0;
        if (lane == src) {
            int cum = excl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (cum + cnt[i] >= need) {
                    digit = 255 - 4 * lane - i;
                    rest = need - cum;
                    break;
                }
                cum += cnt[i];
            }
        }
        digit = __builtin_amdgcn_readlane(digit, src);
        need = __builtin_amdgcn_readlane(rest, src);
        prefix |= (uint32_t)digit << shift;
        wave_lds_sync();
    }
    const uint32_t T = prefix;

    // Ids in ascending order, 64 per round: keep key > T, and the first `need` keys == T.
    int written = 0, eq_seen = 0;
    for (int base = 0; base < nc; base += 64) {
        const int j = base + lane;
        const uint32_t key = j < nc ? keys[j] : 0u;
        const bool eq = j < nc && key == T;
        const uint64_t eq_mask = __ballot(eq);
        const bool take = j < nc && (key > T || (eq && eq_seen + lanes_below(eq_mask) < need));
        const uint64_t take_mask = __ballot(take);
        const int pos = written + lanes_below(take_mask);
        if (take && pos < k) out[pos] = j;
        written += __popcll(take_mask);
        eq_seen += __popcll(eq_mask);
    }
    for (int i = k + lane; i < k_max; i += 64) out[i] = -1;
}

}  // namespace seer

using namespace seer;

extern "C" int seer_select_blocks(const float *scores, const int32_t *seqlens, int B, int H, int nb_max,
                                  int block_size, int budget_tokens, int32_t *block_idx, int32_t *n_sel,
                                  hipStream_t stream) {
    if (!seqlens || !n_sel || B <= 0 || H <= 0 || nb_max < 0 || block_size <= 0 || budget_tokens < 0)
        return SEER_ERR_INVALID_ARG;
    const int k_max = budget_tokens / block_size;
    if ((k_max > 0 && !block_idx) || (nb_max > 0 && !scores)) return SEER_ERR_INVALID_ARG;
    if (nb_max > kSelMaxBlocks) return SEER_ERR_UNSUPPORTED;
    const int64_t pairs = (int64_t)B * H;
    if (pairs > (1LL << 30)) return SEER_ERR_INVALID_ARG;
    // LDS slice per wave: the keys plus a 256-bin histogram; up to 4 waves while it stays within 64 KiB.
    const int slice = nb_max + 256;
    int waves = (int)(65536 / ((size_t)slice * 4));
    waves = waves < 1 ? 1 : (waves > 4 ? 4 : waves);
    const size_t shmem = (size_t)waves * slice * sizeof(uint32_t);
    const int grid = (int)((pairs + waves - 1) / waves);
    select_blocks_kernel<<<dim3(grid), 64 * waves, shmem, stream>>>(scores, seqlens, B, H, nb_max, slice,
                                                                    block_size, k_max, block_idx, n_sel);
    return launch_status();
}
