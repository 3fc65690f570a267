// gate_select.hip -- gate scores and token-budget selection in one launch
// (seer_gate_select): one 1024-thread workgroup per (b, KV head).
//
// With at least a quarter as many (b, KV head) pairs as compute units, one
// workgroup per pair streams the pair's pooled keys and selects from the
// scores held in LDS, with no second launch.  One workgroup per pair keeps
// only that many compute units streaming, so this form takes about as long as
// seer_gate_scores (every compute unit streams) plus seer_select_blocks.  With
// fewer pairs, or shapes outside the limits of the one-workgroup form, the
// call runs those two.
#include "gate_select_items.hpp"
#include "seer_host.hpp"

namespace seer {

constexpr int kGsThreads = 1024;
constexpr int kGsMaxBlocks = 12288;  // LDS keys of one pair (48 KiB) beside the static arrays

template <int D, int G, class KT>
__global__ __launch_bounds__(kGsThreads) void gate_select_kernel(const GateSelectArgs gs) {
    __shared__ GsSmem<D, kGsThreads> sm;
    extern __shared__ uint32_t keys[];
    gate_select_pair<D, G, kGsThreads, LaunchMem, KT>(gs, blockIdx.x, sm, keys);
}

template <int D, class KT>
static void launch_gate_select(const GateSelectArgs &gs, int G, unsigned grid, size_t lds, hipStream_t stream) {
    switch (G) {
        case 1: gate_select_kernel<D, 1, KT><<<grid, kGsThreads, lds, stream>>>(gs); break;
        case 2: gate_select_kernel<D, 2, KT><<<grid, kGsThreads, lds, stream>>>(gs); break;
        case 4: gate_select_kernel<D, 4, KT><<<grid, kGsThreads, lds, stream>>>(gs); break;
        default: gate_select_kernel<D, 8, KT><<<grid, kGsThreads, lds, stream>>>(gs); break;
    }
}

}  // namespace seer

using namespace seer;

extern "C" int seer_gate_select_ex(const seer_bf16 *q, int64_t sq_b, int64_t sq_h, const seer_bf16 *wq,
                                   const seer_bf16 *wk, int dg, const void *kpool, int kpool_dtype, int nb_max,
                                   const int32_t *seqlens, int B, int Hq, int Hkv, int d, int block_size,
                                   float gate_scale, int k_max, const seer_select_policy *policy, float *scores,
                                   int32_t *block_idx, int32_t *n_sel, hipStream_t stream) {
    SelectPolicy pol;
    if (!q || !wq || !wk || !seqlens || !scores || !n_sel) return SEER_ERR_INVALID_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || nb_max < 0 || block_size <= 0 || dg < 1 || dg > 256 ||
        k_max < 0 || !rows_aligned16(q, sq_h) || !rows_aligned16(q, sq_b) || !aligned16(wq) || !aligned16(wk) ||
        !(gate_scale == gate_scale) || !policy_from_host(policy, &pol))
        return SEER_ERR_INVALID_ARG;
    if (k_max > 0 && !block_idx) return SEER_ERR_INVALID_ARG;
    if (nb_max > 0 && (!kpool || !aligned16(kpool))) return SEER_ERR_INVALID_ARG;
    if (kpool_dtype != SEER_KPOOL_F32 && kpool_dtype != SEER_KPOOL_BF16) return SEER_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return SEER_ERR_UNSUPPORTED;
    const int64_t pairs = (int64_t)B * Hkv;
    if (pairs > 65535) return SEER_ERR_INVALID_ARG;
    const int G = Hq / Hkv;
    const bool group_ok = G == 1 || G == 2 || G == 4 || G == 8;
    const bool bf16 = kpool_dtype == SEER_KPOOL_BF16;
    if (bf16 && (!group_ok || nb_max > kGsMaxBlocks)) return SEER_ERR_UNSUPPORTED;  // bf16: one launch only
    const bool one_launch = group_ok && nb_max <= kGsMaxBlocks && (bf16 || 4 * pairs >= device_cu_count());
    if (!one_launch) {
        int st = seer_gate_scores(q, sq_b, sq_h, wq, wk, dg, static_cast<const float *>(kpool), nb_max, seqlens, B,
                                  Hq, Hkv, d, block_size, gate_scale, scores, stream);
        if (st != SEER_OK) return st;
        return seer_select_blocks_ex(scores, seqlens, B, Hkv, nb_max, block_size, k_max, policy, block_idx, n_sel,
                                     stream);
    }
    GateSelectArgs gs{GateArgs{q, sq_b, sq_h, wq, wk, dg, G, Hkv, gate_scale, static_cast<const float *>(kpool), nb_max,
                               seqlens, block_size, scores},
                      pol, k_max, block_idx, n_sel};
    const size_t lds = (size_t)(nb_max > 0 ? nb_max : 1) * sizeof(uint32_t);
    if (d == 128) {
        if (bf16) launch_gate_select<128, uint16_t>(gs, G, (unsigned)pairs, lds, stream);
        else launch_gate_select<128, float>(gs, G, (unsigned)pairs, lds, stream);
    } else {
        if (bf16) launch_gate_select<64, uint16_t>(gs, G, (unsigned)pairs, lds, stream);
        else launch_gate_select<64, float>(gs, G, (unsigned)pairs, lds, stream);
    }
    return launch_status();
}

extern "C" int seer_gate_select(const seer_bf16 *q, int64_t sq_b, int64_t sq_h, const seer_bf16 *wq,
                                const seer_bf16 *wk, int dg, const float *kpool, int nb_max, const int32_t *seqlens,
                                int B, int Hq, int Hkv, int d, int block_size, float gate_scale, int budget_tokens,
                                float *scores, int32_t *block_idx, int32_t *n_sel, hipStream_t stream) {
    if (block_size <= 0 || budget_tokens < 0) return SEER_ERR_INVALID_ARG;
    return seer_gate_select_ex(q, sq_b, sq_h, wq, wk, dg, kpool, SEER_KPOOL_F32, nb_max, seqlens, B, Hq, Hkv, d,
                               block_size, gate_scale, budget_tokens / block_size, nullptr, scores, block_idx, n_sel,
                               stream);
}
