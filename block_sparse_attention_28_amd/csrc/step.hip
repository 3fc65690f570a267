// step.hip -- one gated sparse decode step in two launches.
//
// The same work and results as seer_gate_scores + seer_select_blocks +
// seer_sparse_decode (see gate_items.hpp, topk_block.hpp and decode_items.hpp
// for the operation), with two of their four kernel launches removed:
//
//   1. the gate scores, every compute unit streaming pooled keys (the
//      standalone gate kernel);
//   2. one workgroup per (split, KV head, sequence) that loads its pair's
//      scores into LDS, selects the pair's blocks there (the selection is exact
//      and deterministic, so the S splits of a pair agree; split 0 also writes
//      block_idx and n_sel), decodes its split, and -- the pair's last split to
//      finish -- merges the S partial results.
//
// Each kernel boundary costs several microseconds on this part (dispatch and
// the caches' release / acquire around every launch), about what the
// selection and the merge kernels take in all.  The selection inside the
// decode kernel runs in every workgroup at once, before its first K/V loads;
// the merge hand-off uses device-coherent stores and loads of the split
// partials and one counter per pair.  No workgroup ever waits for another:
// the last split of a pair to bump the counter does the merge, and also
// puts the counter back to zero for the next launch.
#include "decode_items.hpp"
#include "seer_host.hpp"
#include "topk_block.hpp"

#include <hip/hip_runtime.h>

namespace seer {

struct StepArgs {
    DecodeArgs dec;
    const float *scores;  // [B][Hkv][nb_max], written by the gate launch
    int nb_max, block_size;
    int *counters;        // [B * Hkv] merge arrivals, zero between launches
};

template <int D, int BS, int G>
union StepSmem {
    DecodeSmem<D, BS, G> dec;
    MergeSmem merge;
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

// True, in every thread, for the workgroup whose increment brought *ctr to
// `target`: every thread's device-coherent stores have completed before the
// increment, so that workgroup sees every producer's partials.
__device__ __forceinline__ bool arrive_last(int *ctr, int target, int *s_old) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) *s_old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(*s_old) == target - 1;
}

template <int D, int BS, int G>
__global__ __launch_bounds__(256, 2) void decode_select_split_kernel(const StepArgs s) {
    __shared__ StepSmem<D, BS, G> sm;
    extern __shared__ uint32_t keys[];  // selection keys [nb_max], then the kept ids in place
    __shared__ int s_flag;
    const DecodeArgs &a = s.dec;
    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int pair = b * a.Hkv + g, S = a.num_splits;
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

    decode_split_item<D, BS, G, DeviceMem, false, false, true>(a, split, g, b, sm.dec, nullptr, kept, k);

    // The pair's last split to arrive merges the S partial results and puts the
    // pair's counter back to zero for the next launch.
    if (S > 1 && arrive_last(s.counters + pair, S, &s_flag)) {
        if (threadIdx.x == 0) __hip_atomic_store(s.counters + pair, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int h = 0; h < G; ++h)
            decode_merge_row<D, DeviceMem>(a.part_o, a.part_ml, S, (int64_t)b * a.Hq + g * G + h, a.out, a.out_dtype,
                                           a.lse, sm.merge);
    }
}

template <int D, int BS, int G>
static int launch_step_decode(const StepArgs &s, int B, size_t lds, hipStream_t stream) {
    decode_select_split_kernel<D, BS, G><<<dim3(s.dec.num_splits, s.dec.Hkv, B), 256, lds, stream>>>(s);
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

static size_t step_ctl_bytes(int pairs) { return ((size_t)pairs * sizeof(int) + 255) / 256 * 256; }

}  // namespace seer

using namespace seer;

extern "C" size_t seer_decode_step_workspace_size(int B, int Hq, int Hkv, int d, int k_max, int block_size,
                                                  int num_splits) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return 0;
    return step_ctl_bytes(B * Hkv) + seer_sparse_decode_workspace_size(B, Hq, Hkv, d, k_max, block_size, num_splits);
}

extern "C" int seer_decode_step(const seer_bf16 *q, int64_t sq_b, int64_t sq_h, const seer_bf16 *k,
                                const seer_bf16 *v, int64_t skv_b, int64_t skv_h, int64_t skv_t, int kv_capacity,
                                const int32_t *seqlens, const seer_bf16 *wq, const seer_bf16 *wk, int dg,
                                float gate_scale, const float *kpool, int nb_max, int B, int Hq, int Hkv, int d,
                                int block_size, int budget_tokens, float softmax_scale, int num_splits, float *scores,
                                int32_t *block_idx, int32_t *n_sel, void *workspace, size_t workspace_bytes,
                                void *out, int out_dtype, float *lse, hipStream_t stream) {
    // Host-side checks: the union of the three calls this step replaces.
    if (!q || !k || !v || !seqlens || !wq || !wk || !kpool || !scores || !n_sel || !out || !workspace)
        return SEER_ERR_INVALID_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || nb_max <= 0 || budget_tokens < 0 || kv_capacity < 0 ||
        num_splits < 0 || dg < 1 || dg > 256 || !(gate_scale == gate_scale) || !softmax_scale_ok(softmax_scale))
        return SEER_ERR_INVALID_ARG;
    const int k_max = block_size > 0 ? budget_tokens / block_size : 0;
    if (k_max > 0 && !block_idx) return SEER_ERR_INVALID_ARG;
    if (out_dtype != SEER_OUT_BF16 && out_dtype != SEER_OUT_F32) return SEER_ERR_INVALID_ARG;
    if (skv_t < d || !rows_aligned16(q, sq_h) || !rows_aligned16(q, sq_b) || !rows_aligned16(k, skv_t) ||
        !rows_aligned16(v, skv_t) || skv_h % 8 || skv_b % 8 || !aligned16(wq) || !aligned16(wk) || !aligned16(kpool) ||
        !aligned16(workspace))
        return SEER_ERR_INVALID_ARG;
    const int G = Hq / Hkv;
    if ((d != 64 && d != 128) || (block_size != 64 && block_size != 128) || !pow2_group(G) || G > 8)
        return SEER_ERR_UNSUPPORTED;
    if ((int64_t)kv_capacity * skv_t * 2 > 0x7fffffffLL || nb_max > 16384 - 256) return SEER_ERR_UNSUPPORTED;
    const int pairs = B * Hkv;
    if ((int64_t)B * Hkv > 65535) return SEER_ERR_INVALID_ARG;
    const int S = seer_sparse_decode_num_splits(B, Hkv, k_max, block_size, num_splits);
    if (S > kMaxSplits) return SEER_ERR_INVALID_ARG;
    if (workspace_bytes < seer_decode_step_workspace_size(B, Hq, Hkv, d, k_max, block_size, S))
        return SEER_ERR_WORKSPACE;

    // Launch 1: the gate scores.
    int st = seer_gate_scores(q, sq_b, sq_h, wq, wk, dg, kpool, nb_max, seqlens, B, Hq, Hkv, d, block_size,
                              gate_scale, scores, stream);
    if (st != SEER_OK) return st;

    // Launch 2: selection, split decode and merge.
    StepArgs s;
    char *ws = static_cast<char *>(workspace);
    DecodeArgs &a = s.dec;
    a.q = q; a.sq_b = sq_b; a.sq_h = sq_h;
    a.k = k; a.v = v; a.skv_b = skv_b; a.skv_h = skv_h; a.skv_t = skv_t;
    a.kv_capacity = kv_capacity;
    a.seqlens = seqlens; a.block_idx = block_idx; a.n_sel = n_sel;
    a.k_max = k_max; a.Hq = Hq; a.Hkv = Hkv; a.num_splits = S;
    a.scale_log2 = softmax_scale * kLog2e;
    a.part_o = S > 1 ? reinterpret_cast<float *>(ws + step_ctl_bytes(pairs)) : nullptr;
    a.part_ml = S > 1 ? reinterpret_cast<float2 *>(a.part_o + (size_t)B * Hq * S * d) : nullptr;
    a.out = out; a.out_dtype = out_dtype; a.lse = lse;
    a.blk_lse = nullptr; a.units_max = 0;
    s.scores = scores;
    s.nb_max = nb_max;
    s.block_size = block_size;
    s.counters = reinterpret_cast<int *>(ws);
    const size_t lds = (size_t)nb_max * sizeof(uint32_t);
    if (d == 128)
        return block_size == 128 ? step_dispatch_group<128, 128>(s, B, lds, G, stream)
                                 : step_dispatch_group<128, 64>(s, B, lds, G, stream);
    return block_size == 128 ? step_dispatch_group<64, 128>(s, B, lds, G, stream)
                             : step_dispatch_group<64, 64>(s, B, lds, G, stream);
}
