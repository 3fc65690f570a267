// heads.hip -- per-query-head selection (the alternative to one shared block
// set per KV head): gate + per-head selection in one launch, and the sparse
// decode over the union of a group's sets with per-head masks.
//
// Operation: every query head h keeps its own top-k blocks by its own gate
// score (the SeerAttention gate, "SeerAttention: Learning Intrinsic Sparse
// Attention in Your LLMs", abstract v1, without the group mean) and attends
// only those blocks plus the tail ("SeerAttention-R", abstract: sparse
// decoding over the kept blocks).  The decode reads each block of the union
// once for all the group's heads; a head that did not keep a block gives it
// no weight.  Bodies: gate_heads_items.hpp and decode_items.hpp (PH form).
#include "decode_items.hpp"
#include "gate_heads_items.hpp"
#include "seer_host.hpp"

namespace seer {

constexpr int kGhThreads = 1024;
constexpr int kGhMaxKeys = 10240;  // G * nb_max LDS keys of one (b, KV head)
constexpr int kPhMaxBlocks = 4096;  // per-head decode: bitmaps and union in LDS

template <int D, int G>
__global__ __launch_bounds__(kGhThreads) void gate_select_heads_kernel(const GateSelectArgs gs) {
    __shared__ GhSmem<D, kGhThreads, G> sm;
    extern __shared__ uint32_t keys[];
    gate_select_heads_pair<D, G, kGhThreads, LaunchMem>(gs, blockIdx.x, sm, keys);
}

template <int D, int BS, int G>
__global__ __launch_bounds__(256, G >= 8 ? 2 : 3) void sparse_decode_heads_kernel(const DecodeArgs a) {
    __shared__ DecodeSmem<D, BS, G> sm;
    extern __shared__ uint32_t dyn[];
    decode_split_item<D, BS, G, LaunchMem, false, true>(a, blockIdx.x, blockIdx.y, blockIdx.z, sm, dyn);
}

template <int D>
__global__ __launch_bounds__(128) void heads_merge_kernel(const float *part_o, const float2 *part_ml, int S, void *out,
                                                          int out_dtype, float *lse) {
    __shared__ MergeSmem sm;
    decode_merge_row<D, LaunchMem>(part_o, part_ml, S, blockIdx.x, out, out_dtype, lse, sm);
}

template <int D, int BS, int G>
static int launch_heads_decode(const DecodeArgs &a, int B, hipStream_t stream) {
    dim3 grid(a.num_splits, a.Hkv, B);
    const size_t lds = (size_t)heads_union_words(a.units_max, G, a.k_max) * sizeof(uint32_t);
    sparse_decode_heads_kernel<D, BS, G><<<grid, 256, lds, stream>>>(a);
    int st = launch_status();
    if (st != SEER_OK || a.num_splits == 1) return st;
    heads_merge_kernel<D><<<dim3(B * a.Hq), 128, 0, stream>>>(a.part_o, a.part_ml, a.num_splits, a.out, a.out_dtype,
                                                             a.lse);
    return launch_status();
}

template <int D, int BS>
static int dispatch_heads_decode(const DecodeArgs &a, int B, int G, hipStream_t stream) {
    switch (G) {
        case 1: return launch_heads_decode<D, BS, 1>(a, B, stream);
        case 2: return launch_heads_decode<D, BS, 2>(a, B, stream);
        case 4: return launch_heads_decode<D, BS, 4>(a, B, stream);
        case 8: return launch_heads_decode<D, BS, 8>(a, B, stream);
    }
    return SEER_ERR_UNSUPPORTED;
}

}  // namespace seer

using namespace seer;

extern "C" int seer_gate_select_heads(const seer_bf16 *q, int64_t sq_b, int64_t sq_h, const seer_bf16 *wq,
                                      const seer_bf16 *wk, int dg, const float *kpool, int nb_max,
                                      const int32_t *seqlens, int B, int Hq, int Hkv, int d, int block_size,
                                      float gate_scale, int budget_tokens, float *scores, int32_t *block_idx,
                                      int32_t *n_sel, hipStream_t stream) {
    if (!q || !wq || !wk || !seqlens || !scores || !n_sel) return SEER_ERR_INVALID_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || nb_max < 0 || block_size <= 0 || dg < 1 || dg > 256 ||
        budget_tokens < 0 || !rows_aligned16(q, sq_h) || !rows_aligned16(q, sq_b) || !aligned16(wq) ||
        !aligned16(wk) || !(gate_scale == gate_scale))
        return SEER_ERR_INVALID_ARG;
    const int k_max = budget_tokens / block_size;
    if (k_max > 0 && !block_idx) return SEER_ERR_INVALID_ARG;
    if (nb_max > 0 && (!kpool || !aligned16(kpool))) return SEER_ERR_INVALID_ARG;
    const int G = Hq / Hkv;
    if ((d != 64 && d != 128) || !(G == 1 || G == 2 || G == 4 || G == 8) || (int64_t)G * nb_max > kGhMaxKeys)
        return SEER_ERR_UNSUPPORTED;
    const int64_t pairs = (int64_t)B * Hkv;
    if (pairs > 65535) return SEER_ERR_INVALID_ARG;
    GateSelectArgs gs{GateArgs{q, sq_b, sq_h, wq, wk, dg, G, Hkv, gate_scale, kpool, nb_max, seqlens, block_size,
                               scores},
                      SelectPolicy{0, 1, 1, 0.f}, k_max, block_idx, n_sel};
    const size_t lds = (size_t)(G * nb_max > 0 ? G * nb_max : 1) * sizeof(uint32_t);
    const dim3 grid((unsigned)pairs);
#define SEER_GH(D_)                                                                                   \
    switch (G) {                                                                                      \
        case 1: gate_select_heads_kernel<D_, 1><<<grid, kGhThreads, lds, stream>>>(gs); break;        \
        case 2: gate_select_heads_kernel<D_, 2><<<grid, kGhThreads, lds, stream>>>(gs); break;        \
        case 4: gate_select_heads_kernel<D_, 4><<<grid, kGhThreads, lds, stream>>>(gs); break;        \
        default: gate_select_heads_kernel<D_, 8><<<grid, kGhThreads, lds, stream>>>(gs); break;       \
    }
    if (d == 128) {
        SEER_GH(128)
    } else {
        SEER_GH(64)
    }
#undef SEER_GH
    return launch_status();
}

extern "C" size_t seer_sparse_decode_heads_workspace_size(int B, int Hq, int Hkv, int d, int k_max, int nb_max,
                                                          int block_size, int num_splits) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || k_max < 0 || nb_max < 0) return 0;
    const int ku = heads_union_cap(nb_max, Hq / Hkv, k_max);
    return seer_sparse_decode_workspace_size(B, Hq, Hkv, d, ku, block_size, num_splits);
}

extern "C" int seer_sparse_decode_heads(const seer_bf16 *q, int64_t sq_b, int64_t sq_h, const seer_bf16 *k,
                                        const seer_bf16 *v, int64_t skv_b, int64_t skv_h, int64_t skv_t,
                                        int kv_capacity, const int32_t *seqlens, const int32_t *block_idx,
                                        const int32_t *n_sel, int k_max, int nb_max, int B, int Hq, int Hkv, int d,
                                        int block_size, float softmax_scale, int num_splits, void *workspace,
                                        size_t workspace_bytes, void *out, int out_dtype, float *lse,
                                        hipStream_t stream) {
    if (!q || !k || !v || !seqlens || !n_sel || !out) return SEER_ERR_INVALID_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || k_max < 0 || nb_max < 0 || kv_capacity < 0 ||
        num_splits < 0)
        return SEER_ERR_INVALID_ARG;
    if (k_max > 0 && !block_idx) return SEER_ERR_INVALID_ARG;
    if (out_dtype != SEER_OUT_BF16 && out_dtype != SEER_OUT_F32) return SEER_ERR_INVALID_ARG;
    if (skv_t < d || !rows_aligned16(q, sq_h) || !rows_aligned16(q, sq_b) || !rows_aligned16(k, skv_t) ||
        !rows_aligned16(v, skv_t) || skv_h % 8 || skv_b % 8 || !softmax_scale_ok(softmax_scale))
        return SEER_ERR_INVALID_ARG;
    const int G = Hq / Hkv;
    if ((d != 64 && d != 128) || (block_size != 64 && block_size != 128) || !pow2_group(G) || G > 8 ||
        nb_max > kPhMaxBlocks)
        return SEER_ERR_UNSUPPORTED;
    if ((int64_t)kv_capacity * skv_t * 2 > 0x7fffffffLL) return SEER_ERR_UNSUPPORTED;
    const int ku = heads_union_cap(nb_max, G, k_max);
    const int S = seer_sparse_decode_num_splits(B, Hkv, ku, block_size, num_splits);
    if (S > kMaxSplits) return SEER_ERR_INVALID_ARG;
    const size_t need = seer_sparse_decode_workspace_size(B, Hq, Hkv, d, ku, block_size, S);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return SEER_ERR_WORKSPACE;

    DecodeArgs a;
    a.q = q; a.sq_b = sq_b; a.sq_h = sq_h;
    a.k = k; a.v = v; a.skv_b = skv_b; a.skv_h = skv_h; a.skv_t = skv_t;
    a.kv_capacity = kv_capacity;
    a.seqlens = seqlens; a.block_idx = block_idx; a.n_sel = n_sel;
    a.k_max = k_max; a.Hq = Hq; a.Hkv = Hkv; a.num_splits = S;
    a.scale_log2 = softmax_scale * kLog2e;
    a.part_o = static_cast<float *>(workspace);
    a.part_ml = S > 1 ? reinterpret_cast<float2 *>(static_cast<float *>(workspace) + (size_t)B * Hq * S * d) : nullptr;
    a.out = out; a.out_dtype = out_dtype; a.lse = lse;
    a.blk_lse = nullptr; a.units_max = nb_max;
    if (d == 128)
        return block_size == 128 ? dispatch_heads_decode<128, 128>(a, B, G, stream)
                                 : dispatch_heads_decode<128, 64>(a, B, G, stream);
    return block_size == 128 ? dispatch_heads_decode<64, 128>(a, B, G, stream)
                             : dispatch_heads_decode<64, 64>(a, B, G, stream);
}
