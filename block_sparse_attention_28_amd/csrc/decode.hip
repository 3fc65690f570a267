// decode.hip -- split-KV sparse flash-decode over gate-selected KV blocks, and
// the log-sum-exp merge of the splits.
//
// Operation ("SeerAttention-R: Sparse Attention Adaptation for Long
// Reasoning", abstract): a decoding kernel that reads only the KV blocks the
// gate kept.  For sequence b, KV head g and each query head h of g's group,
// softmax attention over T = (kept blocks) + (incomplete tail block).  The
// tail is always attended: it holds the current token and has no pooled key
// to be scored with.
//
// The kernel bodies, and the description of their gfx950 mapping (LDS-direct
// K/V tile loads, both products on v_mfma_f32_16x16x32_bf16 with the group's
// query heads as the N dimension, log2-domain online softmax, per-split
// (o, m, l) partials), are in decode_items.hpp, shared with the decode step
// (step.hip).  This file holds the launches: the split kernel, the log-sum-exp merge
// of the splits, and the dense ground-truth form with its block masses.
#include "decode_items.hpp"

#include <mutex>

namespace seer {

template <int D, int BS, int G>
__global__ __launch_bounds__(256, G >= 8 ? 2 : 3) void sparse_decode_split_kernel(const DecodeArgs a) {
    __shared__ DecodeSmem<D, BS, G> sm;
    decode_split_item<D, BS, G, LaunchMem>(a, blockIdx.x, blockIdx.y, blockIdx.z, sm);
}

template <int D>
__global__ __launch_bounds__(128) void sparse_decode_merge_kernel(const float *part_o, const float2 *part_ml,
                                                                  int S, void *out, int out_dtype, float *lse) {
    __shared__ MergeSmem sm;
    decode_merge_row<D, LaunchMem>(part_o, part_ml, S, blockIdx.x, out, out_dtype, lse, sm);
}

template <int D, int BS, int G>
static int launch_decode(const DecodeArgs &a, int B, hipStream_t stream) {
    dim3 grid(a.num_splits, a.Hkv, B);
    sparse_decode_split_kernel<D, BS, G><<<grid, 256, 0, stream>>>(a);
    int st = launch_status();
    if (st != SEER_OK || a.num_splits == 1) return st;
    sparse_decode_merge_kernel<D><<<dim3(B * a.Hq), 128, 0, stream>>>(a.part_o, a.part_ml, a.num_splits, a.out,
                                                                     a.out_dtype, a.lse);
    return launch_status();
}

// ---------------------------------------------------------- ground truth ----
// Dense form of the split kernel (every complete block, then the tail) that
// also records each unit's per-wave log-sum-exp; then the block masses.
template <int D, int BS, int G>
__global__ __launch_bounds__(256, G >= 8 ? 2 : 3) void block_mass_split_kernel(const DecodeArgs a) {
    __shared__ DecodeSmem<D, BS, G> sm;
    decode_split_item<D, BS, G, LaunchMem, true>(a, blockIdx.x, blockIdx.y, blockIdx.z, sm);
}

// One (b, KV head) per workgroup: mass of unit u = mean over the group's heads
// of 2^(log2-sum-exp of the unit - log2-sum-exp of the whole context).  A
// unit's log2-sum-exp is kept as one entry per 32-token slice (block_size / 32
// of the 4 slots).
template <int G>
__global__ __launch_bounds__(256) void block_mass_kernel(const float *blk_lse, const float *lse, const int32_t *seqlens,
                                                         int Hq, int Hkv, int kv_capacity, int block_size, int nb_max,
                                                         float *mass) {
    const int pair = blockIdx.x, b = pair / Hkv, g = pair % Hkv;
    int L = seqlens[b];
    L = L < 0 ? 0 : (L > kv_capacity ? kv_capacity : L);
    int nc = L / block_size;
    const bool tail = L - nc * block_size > 0;
    nc = nc < nb_max ? nc : nb_max;
    float lse2[G];
#pragma unroll
    for (int h = 0; h < G; ++h) lse2[h] = lse[(int64_t)b * Hq + g * G + h] * kLog2e;
    float *row = mass + (int64_t)pair * (nb_max + 1);
    for (int j = threadIdx.x; j <= nb_max; j += blockDim.x) {
        const int u = j < nc ? j : (j == nb_max && tail ? nc : -1);  // slot nb_max holds the tail
        float m = 0.f;
        if (u >= 0) {
            const float *x = blk_lse + ((int64_t)pair * (nb_max + 1) + u) * G * 4;
            const int nslot = block_size / 32;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = e < nslot ? x[h * 4 + e] : -INFINITY;
                const float mx = fmaxf(fmaxf(w[0], w[1]), fmaxf(w[2], w[3]));
                if (mx == -INFINITY || lse2[h] == -INFINITY) continue;
                float sum = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) sum += exp2f(w[e] - mx);
                m += exp2f(mx + log2f(sum) - lse2[h]);
            }
            m *= 1.0f / (float)G;
        }
        row[j] = m;
    }
}

template <int D, int BS, int G>
static int launch_block_mass(const DecodeArgs &a, int B, const int32_t *seqlens, int block_size, int nb_max,
                             float *mass, hipStream_t stream) {
    dim3 grid(a.num_splits, a.Hkv, B);
    block_mass_split_kernel<D, BS, G><<<grid, 256, 0, stream>>>(a);
    int st = launch_status();
    if (st != SEER_OK) return st;
    if (a.num_splits > 1) {
        sparse_decode_merge_kernel<D><<<dim3(B * a.Hq), 128, 0, stream>>>(a.part_o, a.part_ml, a.num_splits, a.out,
                                                                         a.out_dtype, a.lse);
        if ((st = launch_status()) != SEER_OK) return st;
    }
    block_mass_kernel<G><<<dim3(B * a.Hkv), 256, 0, stream>>>(a.blk_lse, a.lse, seqlens, a.Hq, a.Hkv, a.kv_capacity,
                                                              block_size, nb_max, mass);
    return launch_status();
}

template <int D, int BS>
static int dispatch_block_mass(const DecodeArgs &a, int B, int G, const int32_t *seqlens, int block_size, int nb_max,
                               float *mass, hipStream_t stream) {
    switch (G) {
        case 1: return launch_block_mass<D, BS, 1>(a, B, seqlens, block_size, nb_max, mass, stream);
        case 2: return launch_block_mass<D, BS, 2>(a, B, seqlens, block_size, nb_max, mass, stream);
        case 4: return launch_block_mass<D, BS, 4>(a, B, seqlens, block_size, nb_max, mass, stream);
        case 8: return launch_block_mass<D, BS, 8>(a, B, seqlens, block_size, nb_max, mass, stream);
    }
    return SEER_ERR_UNSUPPORTED;
}

template <int D, int BS>
static int dispatch_group(const DecodeArgs &a, int B, int G, hipStream_t stream) {
    switch (G) {
        case 1: return launch_decode<D, BS, 1>(a, B, stream);
        case 2: return launch_decode<D, BS, 2>(a, B, stream);
        case 4: return launch_decode<D, BS, 4>(a, B, stream);
        case 8: return launch_decode<D, BS, 8>(a, B, stream);
    }
    return SEER_ERR_UNSUPPORTED;
}

}  // namespace seer

using namespace seer;

extern "C" int seer_sparse_decode_num_splits(int B, int Hkv, int k_max, int block_size, int num_splits) {
    if (num_splits > 0) return num_splits < kMaxSplits ? num_splits : kMaxSplits;
    if (B <= 0 || Hkv <= 0 || k_max < 0 || block_size <= 0) return 1;
    // Units per (b, kvh): the kept blocks plus a possible tail.  Long-running
    // workgroups stream best: aim for about two workgroups per compute unit,
    // all resident at once, each with as many units as that leaves.
    const int units = k_max + 1;
    const int cus = device_cu_count();
    const int64_t pairs = (int64_t)B * Hkv;
    int64_t s = (2LL * cus + pairs - 1) / pairs;
    if (s > units) s = units;
    if (s > kMaxSplits) s = kMaxSplits;
    return s < 1 ? 1 : (int)s;
}

extern "C" size_t seer_sparse_decode_workspace_size(int B, int Hq, int Hkv, int d, int k_max, int block_size,
                                                    int num_splits) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return 0;
    const int s = seer_sparse_decode_num_splits(B, Hkv, k_max, block_size, num_splits);
    if (s <= 1) return 0;
    return (size_t)B * Hq * s * ((size_t)d + 2) * sizeof(float);
}

// ------------------------------------------------- allocation-free form ----
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc): the split partials live in
// this file-scope device array instead of a caller workspace.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[SEER_NOALLOC_SCRATCH_BYTES];

namespace seer {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, or null if the lookup failed.
static void *scratch_device_ptr() {
    static std::mutex mu;
    static void *ptrs[kMaxDevices] = {nullptr};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        ptrs[dev] = p;
    }
    return ptrs[dev];
}

// Validation and launch shared by seer_sparse_decode and its allocation-free form;
// `partials` (a caller workspace, or the static scratch) holds `ws_bytes` bytes.
static int sparse_decode_impl(const seer_bf16 *q, int64_t sq_b, int64_t sq_h, const seer_bf16 *k,
                              const seer_bf16 *v, int64_t skv_b, int64_t skv_h, int64_t skv_t, int kv_capacity,
                              const int32_t *seqlens, const int32_t *block_idx, const int32_t *n_sel, int k_max,
                              int B, int Hq, int Hkv, int d, int block_size, float softmax_scale, int num_splits,
                              void *workspace, size_t workspace_bytes, bool static_scratch, void *out,
                              int out_dtype, float *lse, hipStream_t stream) {
    if (!q || !k || !v || !seqlens || !n_sel || !out) return SEER_ERR_INVALID_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || k_max < 0 || kv_capacity < 0 || num_splits < 0)
        return SEER_ERR_INVALID_ARG;
    if (k_max > 0 && !block_idx) return SEER_ERR_INVALID_ARG;
    if (out_dtype != SEER_OUT_BF16 && out_dtype != SEER_OUT_F32) return SEER_ERR_INVALID_ARG;
    if (skv_t < d || !rows_aligned16(q, sq_h) || !rows_aligned16(q, sq_b) || !rows_aligned16(k, skv_t) ||
        !rows_aligned16(v, skv_t) || skv_h % 8 || skv_b % 8 || !softmax_scale_ok(softmax_scale))
        return SEER_ERR_INVALID_ARG;
    const int G = Hq / Hkv;
    if ((d != 64 && d != 128) || (block_size != 64 && block_size != 128) || !pow2_group(G) || G > 8)
        return SEER_ERR_UNSUPPORTED;
    const int S = seer_sparse_decode_num_splits(B, Hkv, k_max, block_size, num_splits);
    const size_t need = seer_sparse_decode_workspace_size(B, Hq, Hkv, d, k_max, block_size, S);
    if (static_scratch) {
        if (need > SEER_NOALLOC_SCRATCH_BYTES) return SEER_ERR_WORKSPACE;
        if (need > 0) {
            workspace = scratch_device_ptr();
            if (!workspace) return SEER_ERR_LAUNCH;
            workspace_bytes = SEER_NOALLOC_SCRATCH_BYTES;
        }
    }
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return SEER_ERR_WORKSPACE;
    if (S > kMaxSplits) return SEER_ERR_INVALID_ARG;
    if ((int64_t)kv_capacity * skv_t * 2 > 0x7fffffffLL) return SEER_ERR_UNSUPPORTED;  // buffer offsets are 32-bit

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
    a.blk_lse = nullptr; a.units_max = 0;
    if (d == 128) return block_size == 128 ? dispatch_group<128, 128>(a, B, G, stream) : dispatch_group<128, 64>(a, B, G, stream);
    return block_size == 128 ? dispatch_group<64, 128>(a, B, G, stream) : dispatch_group<64, 64>(a, B, G, stream);
}

}  // namespace seer

extern "C" int seer_sparse_decode(const seer_bf16 *q, int64_t sq_b, int64_t sq_h, const seer_bf16 *k,
                                  const seer_bf16 *v, int64_t skv_b, int64_t skv_h, int64_t skv_t, int kv_capacity,
                                  const int32_t *seqlens, const int32_t *block_idx, const int32_t *n_sel, int k_max,
                                  int B, int Hq, int Hkv, int d, int block_size, float softmax_scale, int num_splits,
                                  void *workspace, size_t workspace_bytes, void *out, int out_dtype, float *lse,
                                  hipStream_t stream) {
    return sparse_decode_impl(q, sq_b, sq_h, k, v, skv_b, skv_h, skv_t, kv_capacity, seqlens, block_idx, n_sel,
                              k_max, B, Hq, Hkv, d, block_size, softmax_scale, num_splits, workspace,
                              workspace_bytes, false, out, out_dtype, lse, stream);
}

extern "C" int seer_sparse_decode_noalloc(const seer_bf16 *q, int64_t sq_b, int64_t sq_h, const seer_bf16 *k,
                                          const seer_bf16 *v, int64_t skv_b, int64_t skv_h, int64_t skv_t,
                                          int kv_capacity, const int32_t *seqlens, const int32_t *block_idx,
                                          const int32_t *n_sel, int k_max, int B, int Hq, int Hkv, int d,
                                          int block_size, float softmax_scale, int num_splits, void *out,
                                          int out_dtype, float *lse, hipStream_t stream) {
    return sparse_decode_impl(q, sq_b, sq_h, k, v, skv_b, skv_h, skv_t, kv_capacity, seqlens, block_idx, n_sel,
                              k_max, B, Hq, Hkv, d, block_size, softmax_scale, num_splits, nullptr, 0, true, out,
                              out_dtype, lse, stream);
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

extern "C" size_t seer_decode_block_mass_workspace_size(int B, int Hq, int Hkv, int d, int nb_max, int block_size,
                                                        int num_splits) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || nb_max < 0 || Hq % Hkv != 0) return 0;
    const int S = seer_sparse_decode_num_splits(B, Hkv, nb_max, block_size, num_splits);
    const size_t parts = align256(seer_sparse_decode_workspace_size(B, Hq, Hkv, d, nb_max, block_size, S));
    const size_t lse = align256((size_t)B * Hq * sizeof(float));
    const size_t blk = (size_t)B * Hq * ((size_t)nb_max + 1) * 4 * sizeof(float);
    return parts + lse + blk;
}

extern "C" int seer_decode_block_mass(const seer_bf16 *q, int64_t sq_b, int64_t sq_h, const seer_bf16 *k,
                                      const seer_bf16 *v, int64_t skv_b, int64_t skv_h, int64_t skv_t,
                                      int kv_capacity, const int32_t *seqlens, int B, int Hq, int Hkv, int d,
                                      int block_size, float softmax_scale, int nb_max, int num_splits,
                                      void *workspace, size_t workspace_bytes, void *out, int out_dtype, float *lse,
                                      float *mass, hipStream_t stream) {
    if (!q || !k || !v || !seqlens || !out || !mass || !workspace) return SEER_ERR_INVALID_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || nb_max < 0 || kv_capacity < 0 || num_splits < 0)
        return SEER_ERR_INVALID_ARG;
    if (out_dtype != SEER_OUT_BF16 && out_dtype != SEER_OUT_F32) return SEER_ERR_INVALID_ARG;
    if (skv_t < d || !rows_aligned16(q, sq_h) || !rows_aligned16(q, sq_b) || !rows_aligned16(k, skv_t) ||
        !rows_aligned16(v, skv_t) || skv_h % 8 || skv_b % 8 || !softmax_scale_ok(softmax_scale) ||
        !aligned16(workspace))
        return SEER_ERR_INVALID_ARG;
    const int G = Hq / Hkv;
    if ((d != 64 && d != 128) || (block_size != 64 && block_size != 128) || !pow2_group(G) || G > 8)
        return SEER_ERR_UNSUPPORTED;
    if ((int64_t)kv_capacity * skv_t * 2 > 0x7fffffffLL) return SEER_ERR_UNSUPPORTED;
    const int S = seer_sparse_decode_num_splits(B, Hkv, nb_max, block_size, num_splits);
    if (S > kMaxSplits) return SEER_ERR_INVALID_ARG;
    if (workspace_bytes < seer_decode_block_mass_workspace_size(B, Hq, Hkv, d, nb_max, block_size, S))
        return SEER_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    const size_t parts = align256(seer_sparse_decode_workspace_size(B, Hq, Hkv, d, nb_max, block_size, S));
    const size_t lse_bytes = align256((size_t)B * Hq * sizeof(float));

    DecodeArgs a;
    a.q = q; a.sq_b = sq_b; a.sq_h = sq_h;
    a.k = k; a.v = v; a.skv_b = skv_b; a.skv_h = skv_h; a.skv_t = skv_t;
    a.kv_capacity = kv_capacity;
    a.seqlens = seqlens; a.block_idx = nullptr; a.n_sel = nullptr;
    a.k_max = nb_max; a.Hq = Hq; a.Hkv = Hkv; a.num_splits = S;
    a.scale_log2 = softmax_scale * kLog2e;
    a.part_o = S > 1 ? reinterpret_cast<float *>(ws) : nullptr;
    a.part_ml = S > 1 ? reinterpret_cast<float2 *>(reinterpret_cast<float *>(ws) + (size_t)B * Hq * S * d) : nullptr;
    a.out = out; a.out_dtype = out_dtype;
    a.lse = lse ? lse : reinterpret_cast<float *>(ws + parts);
    a.blk_lse = reinterpret_cast<float *>(ws + parts + lse_bytes);
    a.units_max = nb_max + 1;
    if (d == 128)
        return block_size == 128 ? dispatch_block_mass<128, 128>(a, B, G, seqlens, block_size, nb_max, mass, stream)
                                 : dispatch_block_mass<128, 64>(a, B, G, seqlens, block_size, nb_max, mass, stream);
    return block_size == 128 ? dispatch_block_mass<64, 128>(a, B, G, seqlens, block_size, nb_max, mass, stream)
                             : dispatch_block_mass<64, 64>(a, B, G, seqlens, block_size, nb_max, mass, stream);
}
