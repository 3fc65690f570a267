// step.hip -- one gated sparse decode step in three launches.
//
// The same work and results as seer_gate_scores + seer_select_blocks +
// seer_sparse_decode (see gate_items.hpp, topk_block.hpp and decode_items.hpp
// for the operation), with the selection's own launch removed:
//
//   1. the gate scores, every compute unit streaming pooled keys (the
//      standalone gate kernel);
//   2. one workgroup per (split, KV head, sequence) that loads its pair's
//      scores into LDS, selects the pair's blocks there (the selection is exact
//      and deterministic, so the S splits of a pair agree; split 0 also writes
//      block_idx and n_sel) and decodes its split;
//   3. the log-sum-exp merge of the splits.
//
// A kernel boundary costs several microseconds on this part (dispatch and the
// caches' release / acquire around every launch); the selection inside the
// decode kernel runs in every workgroup at once, before its first K/V loads,
// and costs less.  The merge stays a launch of its own: merging by the last
// split of each pair inside the decode kernel (device-coherent partials and a
// counter per pair) lengthened the decode's tail by more than a launch costs.
#include "decode_items.hpp"
#include "seer_host.hpp"
#include "topk_block.hpp"

#include <hip/hip_runtime.h>

namespace seer {

struct StepArgs {
    DecodeArgs dec;
    const float *scores;  // [B][Hkv][nb_max], written by the gate launch
    int nb_max, block_size;
};

template <int D, int BS, int G>
union StepSmem {
    DecodeSmem<D, BS, G> dec;
    SelBlockSmem<256> sel;
};

// Scores [0, nc) of one pair as selection keys in LDS; rows past nc read as zero.
__device__ __forceinline__ void load_score_keys(const float *row, int nc, uint32_t *keys) {
    const auto rs = buffer_rsrc(row, (uint32_t)nc * 4);
    for (int j0 = 0; j0 < nc; j0 += 4 * 256) {
        uint32_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, (j0 + i * 256 + (int)threadIdx.x) * 4, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = j0 + i * 256 + (int)threadIdx.x;
            if (j < nc) keys[j] = order_key(__uint_as_float(v[i]));
        }
    }
}

template <int D, int BS, int G>
__global__ __launch_bounds__(256, 2) void decode_select_split_kernel(const StepArgs s) {
    __shared__ StepSmem<D, BS, G> sm;
    extern __shared__ uint32_t keys[];  // selection keys [nb_max], then the kept ids in place
    const DecodeArgs &a = s.dec;
    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int pair = b * a.Hkv + g;
    int L = a.seqlens[b];
    L = L < 0 ? 0 : L;
    int nc = L / s.block_size;
    nc = nc > s.nb_max ? s.nb_max : nc;
    nc = __builtin_amdgcn_readfirstlane(nc);

    // The pair's selection, exactly as seer_select_blocks makes it.
    load_score_keys(s.scores + (int64_t)pair * s.nb_max, nc, keys);
    block_select_prepare<256>(sm.sel);
    __syncthreads();  // keys complete
    int32_t *kept = reinterpret_cast<int32_t *>(keys);
    int32_t *row_out = split == 0 ? const_cast<int32_t *>(a.block_idx) + (int64_t)pair * a.k_max : nullptr;
    const int k = block_select_keys<256, LaunchMem, 2>(keys, nc, SelectPolicy{0, 1, 1, 0.f}, a.k_max, row_out, kept,
                                                      sm.sel);
    if (split == 0 && threadIdx.x == 0) const_cast<int32_t *>(a.n_sel)[pair] = k;
    __syncthreads();  // kept ids complete; the selection's LDS is free for the decode tiles

    decode_split_item<D, BS, G, LaunchMem, false, false, true>(a, split, g, b, sm.dec, nullptr, kept, k);
}

template <int D>
__global__ __launch_bounds__(128) void step_merge_kernel(const float *part_o, const float2 *part_ml, int S, void *out,
                                                         int out_dtype, float *lse) {
    __shared__ MergeSmem sm;
    decode_merge_row<D, LaunchMem>(part_o, part_ml, S, blockIdx.x, out, out_dtype, lse, sm);
}

template <int D, int BS, int G>
static int launch_step_decode(const StepArgs &s, int B, size_t lds, hipStream_t stream) {
    const DecodeArgs &a = s.dec;
    decode_select_split_kernel<D, BS, G><<<dim3(a.num_splits, a.Hkv, B), 256, lds, stream>>>(s);
    int st = launch_status();
    if (st != SEER_OK || a.num_splits == 1) return st;
    step_merge_kernel<D><<<dim3(B * a.Hq), 128, 0, stream>>>(a.part_o, a.part_ml, a.num_splits, a.out, a.out_dtype,
                                                             a.lse);
    return launch_status();
}

template <int D, int BS>
static int step_dispatch_group(const StepArgs &s, int B, size_t lds, int G, hipStream_t stream) {
    switch (G) {
        case 1: return launch_step_decode<D, BS, 1>(s, B, lds, stream);
        case 2: return launch_step_decode<D, BS, 2>(s, B, lds, stream);
        case 4: return launch_step_decode<D, BS, 4>(s, B, lds, stream);
        case 8: return launch_step_decode<D, BS, 8>(s, B, lds, stream);
    }
    return SEER_ERR_UNSUPPORTED;
}

// Checks and arguments of launches 2 and 3 (selection + split decode, merge);
// the kernels' dynamic LDS is the selection keys.
static int select_decode_prepare(const seer_bf16 *q, int64_t sq_b, int64_t sq_h, const seer_bf16 *k,
                                 const seer_bf16 *v, int64_t skv_b, int64_t skv_h, int64_t skv_t, int kv_capacity,
                                 const int32_t *seqlens, const float *scores, int nb_max, int B, int Hq, int Hkv, int d,
                                 int block_size, int budget_tokens, float softmax_scale, int num_splits,
                                 int32_t *block_idx, int32_t *n_sel, void *workspace, size_t workspace_bytes,
                                 void *out, int out_dtype, float *lse, StepArgs &s) {
    if (!q || !k || !v || !seqlens || !scores || !n_sel || !out) return SEER_ERR_INVALID_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || nb_max <= 0 || budget_tokens < 0 || kv_capacity < 0 ||
        num_splits < 0 || !softmax_scale_ok(softmax_scale))
        return SEER_ERR_INVALID_ARG;
    const int k_max = block_size > 0 ? budget_tokens / block_size : 0;
    if (k_max > 0 && !block_idx) return SEER_ERR_INVALID_ARG;
    if (out_dtype != SEER_OUT_BF16 && out_dtype != SEER_OUT_F32) return SEER_ERR_INVALID_ARG;
    if (skv_t < d || !rows_aligned16(q, sq_h) || !rows_aligned16(q, sq_b) || !rows_aligned16(k, skv_t) ||
        !rows_aligned16(v, skv_t) || skv_h % 8 || skv_b % 8)
        return SEER_ERR_INVALID_ARG;
    const int G = Hq / Hkv;
    if ((d != 64 && d != 128) || (block_size != 64 && block_size != 128) || !pow2_group(G) || G > 8)
        return SEER_ERR_UNSUPPORTED;
    if ((int64_t)kv_capacity * skv_t * 2 > 0x7fffffffLL || nb_max > 16384 - 256) return SEER_ERR_UNSUPPORTED;
    if ((int64_t)B * Hkv > 65535) return SEER_ERR_INVALID_ARG;
    const int S = seer_sparse_decode_num_splits(B, Hkv, k_max, block_size, num_splits);
    if (S > kMaxSplits) return SEER_ERR_INVALID_ARG;
    const size_t need = seer_sparse_decode_workspace_size(B, Hq, Hkv, d, k_max, block_size, S);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return SEER_ERR_WORKSPACE;

    float *ws = static_cast<float *>(workspace);
    DecodeArgs &a = s.dec;
    a.q = q; a.sq_b = sq_b; a.sq_h = sq_h;
    a.k = k; a.v = v; a.skv_b = skv_b; a.skv_h = skv_h; a.skv_t = skv_t;
    a.kv_capacity = kv_capacity;
    a.seqlens = seqlens; a.block_idx = block_idx; a.n_sel = n_sel;
    a.k_max = k_max; a.Hq = Hq; a.Hkv = Hkv; a.num_splits = S;
    a.scale_log2 = softmax_scale * kLog2e;
    a.part_o = S > 1 ? ws : nullptr;
    a.part_ml = S > 1 ? reinterpret_cast<float2 *>(ws + (size_t)B * Hq * S * d) : nullptr;
    a.out = out; a.out_dtype = out_dtype; a.lse = lse;
    a.blk_lse = nullptr; a.units_max = 0;
    s.scores = scores;
    s.nb_max = nb_max;
    s.block_size = block_size;
    return SEER_OK;
}

static int select_decode_launch(const StepArgs &s, int B, int d, int block_size, hipStream_t stream) {
    const size_t lds = (size_t)s.nb_max * sizeof(uint32_t);
    const int G = s.dec.Hq / s.dec.Hkv;
    if (d == 128)
        return block_size == 128 ? step_dispatch_group<128, 128>(s, B, lds, G, stream)
                                 : step_dispatch_group<128, 64>(s, B, lds, G, stream);
    return block_size == 128 ? step_dispatch_group<64, 128>(s, B, lds, G, stream)
                             : step_dispatch_group<64, 64>(s, B, lds, G, stream);
}

}  // namespace seer

using namespace seer;

extern "C" int seer_select_sparse_decode(const seer_bf16 *q, int64_t sq_b, int64_t sq_h, const seer_bf16 *k,
                                         const seer_bf16 *v, int64_t skv_b, int64_t skv_h, int64_t skv_t,
                                         int kv_capacity, const int32_t *seqlens, const float *scores, int nb_max,
                                         int B, int Hq, int Hkv, int d, int block_size, int budget_tokens,
                                         float softmax_scale, int num_splits, int32_t *block_idx, int32_t *n_sel,
                                         void *workspace, size_t workspace_bytes, void *out, int out_dtype,
                                         float *lse, hipStream_t stream) {
    StepArgs s;
    const int st = select_decode_prepare(q, sq_b, sq_h, k, v, skv_b, skv_h, skv_t, kv_capacity, seqlens, scores,
                                         nb_max, B, Hq, Hkv, d, block_size, budget_tokens, softmax_scale, num_splits,
                                         block_idx, n_sel, workspace, workspace_bytes, out, out_dtype, lse, s);
    return st != SEER_OK ? st : select_decode_launch(s, B, d, block_size, stream);
}

extern "C" size_t seer_decode_step_workspace_size(int B, int Hq, int Hkv, int d, int k_max, int block_size,
                                                  int num_splits) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return 0;
    return seer_sparse_decode_workspace_size(B, Hq, Hkv, d, k_max, block_size, num_splits);
}

extern "C" int seer_decode_step(const seer_bf16 *q, int64_t sq_b, int64_t sq_h, const seer_bf16 *k,
                                const seer_bf16 *v, int64_t skv_b, int64_t skv_h, int64_t skv_t, int kv_capacity,
                                const int32_t *seqlens, const seer_bf16 *wq, const seer_bf16 *wk, int dg,
                                float gate_scale, const float *kpool, int nb_max, int B, int Hq, int Hkv, int d,
                                int block_size, int budget_tokens, float softmax_scale, int num_splits, float *scores,
                                int32_t *block_idx, int32_t *n_sel, void *workspace, size_t workspace_bytes,
                                void *out, int out_dtype, float *lse, hipStream_t stream) {
    // Every check of both parts before the first launch.
    if (!wq || !wk || !kpool) return SEER_ERR_INVALID_ARG;
    if (dg < 1 || dg > 256 || !(gate_scale == gate_scale) || !aligned16(wq) || !aligned16(wk) || !aligned16(kpool))
        return SEER_ERR_INVALID_ARG;
    StepArgs s;
    int st = select_decode_prepare(q, sq_b, sq_h, k, v, skv_b, skv_h, skv_t, kv_capacity, seqlens, scores, nb_max, B,
                                   Hq, Hkv, d, block_size, budget_tokens, softmax_scale, num_splits, block_idx, n_sel,
                                   workspace, workspace_bytes, out, out_dtype, lse, s);
    if (st != SEER_OK) return st;
    // Launch 1: the gate scores.
    st = seer_gate_scores(q, sq_b, sq_h, wq, wk, dg, kpool, nb_max, seqlens, B, Hq, Hkv, d, block_size, gate_scale,
                          scores, stream);
    if (st != SEER_OK) return st;
    // Launches 2 and 3: selection and split decode, then the merge.
    return select_decode_launch(s, B, d, block_size, stream);
}
