// select.hip -- token-budget top-k block selection.
//
// Operation ("SeerAttention-R: Sparse Attention Adaptation for Long
// Reasoning", abstract: a fixed token budget at 64/128-token block
// granularity): per (sequence, KV head) keep k = min(budget / bs, nc) complete
// blocks with the largest gate scores, equal scores ordered by the lower block
// id, and emit the kept ids in ascending order (so decoding reads memory
// forward).
//
// One 256-thread workgroup per (b, head): the scores go to LDS as
// order-preserving keys and the block-wide selection of topk_block.hpp picks
// from them (the rule itself is stated in topk_wave.hpp).
#include "seer_device.hpp"
#include "seer_host.hpp"
#include "topk_block.hpp"

namespace seer {

constexpr int kSelThreads = 256;
constexpr int kSelMaxBlocks = 16384 - 256;  // LDS keys of one pair (64 KiB less a histogram's worth)

__global__ __launch_bounds__(kSelThreads) void select_blocks_kernel(const float *scores, const int32_t *seqlens,
                                                                    int H, int nb_max, int block_size, int k_max,
                                                                    int32_t *block_idx, int32_t *n_sel,
                                                                    const SelectPolicy pol) {
    extern __shared__ uint32_t keys[];  // [nb_max]
    __shared__ SelBlockSmem<kSelThreads> sm;
    const int pair = blockIdx.x;  // b * H + h
    int L = seqlens[pair / H];
    L = L < 0 ? 0 : L;
    int nc = L / block_size;
    nc = nc > nb_max ? nb_max : nc;
    nc = __builtin_amdgcn_readfirstlane(nc);
    // Four loads per thread in flight; rows past nc read as zero.
    const auto rs = buffer_rsrc(scores + (int64_t)pair * nb_max, (uint32_t)nc * 4);
    for (int j0 = 0; j0 < nc; j0 += 4 * kSelThreads) {
        uint32_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, (j0 + i * kSelThreads + (int)threadIdx.x) * 4, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = j0 + i * kSelThreads + (int)threadIdx.x;
            if (j < nc) keys[j] = order_key(__uint_as_float(v[i]));
        }
    }
    block_select_prepare<kSelThreads>(sm);
    __syncthreads();  // keys complete
    const int k = block_select_keys<kSelThreads, LaunchMem>(keys, nc, pol, k_max, block_idx + (int64_t)pair * k_max,
                                                            nullptr, sm);
    if (threadIdx.x == 0) n_sel[pair] = k;
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
    if (pairs > 0x7fffffffLL) return SEER_ERR_INVALID_ARG;
    const size_t shmem = (size_t)nb_max * sizeof(uint32_t);
    select_blocks_kernel<<<dim3((unsigned)pairs), kSelThreads, shmem, stream>>>(scores, seqlens, H, nb_max, block_size,
                                                                               k_max, block_idx, n_sel, pol);
    return launch_status();
}

extern "C" int seer_select_blocks(const float *scores, const int32_t *seqlens, int B, int H, int nb_max,
                                  int block_size, int budget_tokens, int32_t *block_idx, int32_t *n_sel,
                                  hipStream_t stream) {
    if (block_size <= 0 || budget_tokens < 0) return SEER_ERR_INVALID_ARG;
    return seer_select_blocks_ex(scores, seqlens, B, H, nb_max, block_size, budget_tokens / block_size, nullptr,
                                 block_idx, n_sel, stream);
}
