// select.hip -- token-budget top-k block selection.
//
// Operation ("SeerAttention-R: Sparse Attention Adaptation for Long
// Reasoning", abstract: a fixed token budget at 64/128-token block
// granularity): per (sequence, KV head) keep k = min(budget / bs, nc) complete
// blocks with the largest gate scores, equal scores ordered by the lower block
// id, and emit the kept ids in ascending order (so decoding reads memory
// forward).
//
// One wavefront per (b, head), several per workgroup, no workgroup barriers;
// the exact radix top-k itself is in topk_wave.hpp.
#include "seer_device.hpp"
#include "seer_host.hpp"
#include "topk_wave.hpp"

namespace seer {

constexpr int kSelMaxBlocks = 16384 - 256;  // keys + histogram of one wave fit in 64 KiB of LDS

__global__ __launch_bounds__(256) void select_blocks_kernel(const float *scores, const int32_t *seqlens, int B,
                                                            int H, int nb_max, int slice, int block_size, int k_max,
                                                            int32_t *block_idx, int32_t *n_sel,
                                                            const SelectPolicy pol) {
    extern __shared__ uint32_t lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pair = blockIdx.x * (blockDim.x >> 6) + wave;  // b * H + h
    if (pair >= B * H) return;
    uint32_t *keys = lds + (size_t)wave * slice;              // [nb_max]
    int *hist = reinterpret_cast<int *>(keys + slice - 256);  // [256]

    select_pair_item<LaunchMem>(scores, seqlens, H, nb_max, block_size, k_max, block_idx, n_sel, pair, keys, hist,
                                lane, pol);
}

// Host-side check of a selection policy; NULL means the token budget.
bool policy_from_host(const seer_select_policy *p, SelectPolicy *out) {
    SelectPolicy r{SEER_SELECT_BUDGET, 1, 1, 0.f};
    if (p) {
        if (p->kind != SEER_SELECT_BUDGET && p->kind != SEER_SELECT_RATIO && p->kind != SEER_SELECT_THRESHOLD)
            return false;
        if (p->kind == SEER_SELECT_RATIO && (p->ratio_num < 0 || p->ratio_den <= 0)) return false;
        if (p->kind == SEER_SELECT_THRESHOLD && !(p->threshold == p->threshold)) return false;
        r = SelectPolicy{p->kind, p->ratio_num, p->ratio_den, p->threshold};
    }
    *out = r;
    return true;
}

}  // namespace seer

using namespace seer;

extern "C" int seer_select_blocks_ex(const float *scores, const int32_t *seqlens, int B, int H, int nb_max,
                                     int block_size, int k_max, const seer_select_policy *policy, int32_t *block_idx,
                                     int32_t *n_sel, hipStream_t stream) {
    SelectPolicy pol;
    if (!seqlens || !n_sel || B <= 0 || H <= 0 || nb_max < 0 || block_size <= 0 || k_max < 0 ||
        !policy_from_host(policy, &pol))
        return SEER_ERR_INVALID_ARG;
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
                                                                    block_size, k_max, block_idx, n_sel, pol);
    return launch_status();
}

extern "C" int seer_select_blocks(const float *scores, const int32_t *seqlens, int B, int H, int nb_max,
                                  int block_size, int budget_tokens, int32_t *block_idx, int32_t *n_sel,
                                  hipStream_t stream) {
    if (block_size <= 0 || budget_tokens < 0) return SEER_ERR_INVALID_ARG;
    return seer_select_blocks_ex(scores, seqlens, B, H, nb_max, block_size, budget_tokens / block_size, nullptr,
                                 block_idx, n_sel, stream);
}
