// step.hip -- one gated sparse decode step in a single persistent launch.
//
// The same work as seer_gate_scores + seer_select_blocks + seer_sparse_decode
// (gate rows, per-(b, KV head) selection, decode splits, log-sum-exp merges;
// see gate_items.hpp, topk_block.hpp and decode_items.hpp for the operation),
// but run by one grid of resident workgroups: workgroup w takes work items
// w, w + grid, w + 2 grid, ... in increasing order.  Item (pair, split) for
// split < S does all of that split's work: its share of the pair's gate rows
// (the complete blocks dealt evenly over the S splits), then -- once the
// pair's S shares are in -- the pair's selection, which every split computes
// itself in LDS (it is exact and deterministic, so the S splits agree; split 0
// also writes it out), then the split's decode; the pair's last split to
// finish merges the S partial results.  The grid is a multiple of S, so the S
// items of a pair always run in the same round, on workgroups that are
// resident together (the grid is sized from the occupancy of this kernel), and
// no other wait exists: no deadlock, and every workgroup has the same work.
//
// Hand-offs between workgroups (scores, split partials) use device-coherent
// loads and stores (the workgroups may sit on different XCDs with separate
// L2s); a producer waits for its stores to complete before bumping the item's
// counter, a consumer polls that counter.  Every poll loop has a limit and a
// shared abort word, so a launch always terminates; the last workgroup out
// clears the counters for the next launch.
#include "decode_items.hpp"
#include "gate_items.hpp"
#include "seer_host.hpp"
#include "topk_block.hpp"

#include <hip/hip_runtime.h>

namespace seer {

// Control words at the head of the workspace.
enum : int { kCtlFinished = 1, kCtlStatus = 2, kCtlWords = 4 };
constexpr int kSpinLimit = 1 << 22;

struct StepArgs {
    GateArgs gate;
    DecodeArgs dec;
    int pairs;        // B * Hkv
    int k_max;
    int *ctl;         // [kCtlWords + 2 * pairs]
    int total;            // pairs * S items
};

__device__ __forceinline__ int ld_dev(int *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// Wave 0 polls until *ctr >= target (or the launch was aborted); then the
// workgroup proceeds.  Every decision is made on wave-uniform values so that
// the compiler keeps the workgroup's control flow uniform around the barriers.
__device__ __forceinline__ void wait_for(int *ctr, int target, int *status) {
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0) {
        for (int spins = 0;; ++spins) {
            if (__builtin_amdgcn_readfirstlane(ld_dev(ctr)) >= target) break;
            if (__builtin_amdgcn_readfirstlane(ld_dev(status)) != 0) break;
            if (spins >= kSpinLimit) {
                __hip_atomic_store(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
}

// The scores [0, nc) of a pair as selection keys in LDS: device-coherent (sc1)
// buffer loads, four per thread in flight; rows past nc read as zero.
constexpr int kCoherentLoad = 16;  // cache policy: sc1
__device__ __forceinline__ void load_keys(const float *row, int nc, uint32_t *keys) {
    const auto rs = buffer_rsrc(row, (uint32_t)nc * 4);
    for (int j0 = 0; j0 < nc; j0 += 4 * 256) {
        uint32_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, (j0 + i * 256 + (int)threadIdx.x) * 4, 0, kCoherentLoad);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = j0 + i * 256 + (int)threadIdx.x;
            if (j < nc) keys[j] = order_key(__uint_as_float(v[i]));
        }
    }
}

// As signal_done; true, in every thread, for the workgroup whose increment
// brought the counter to `target` (every other producer's stores are then
// complete and visible).
__device__ __forceinline__ bool signal_done_last(int *ctr, int target, int *s_old) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) *s_old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(*s_old) == target - 1;
}

// Every thread's device-coherent stores of this item have completed; then one increment.
__device__ __forceinline__ void signal_done(int *ctr) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int BS, int G>
union StepSmem {
    DecodeSmem<D, BS, G> dec;
    GateSmem<D> gate;
    MergeSmem merge;
    SelBlockSmem<256> sel;
};

template <int D, int BS, int G>
__global__ __launch_bounds__(256, 2) void decode_step_kernel(const StepArgs s) {
    __shared__ StepSmem<D, BS, G> sm;
    extern __shared__ uint32_t keys[];  // selection keys [nb_max], then the kept ids in place
    int *ctl = s.ctl;
    int *gate_done = ctl + kCtlWords, *dec_done = gate_done + s.pairs;
    int *status = ctl + kCtlStatus;
    const int S = s.dec.num_splits, Hkv = s.dec.Hkv, nb_max = s.gate.nb_max;
    __shared__ int s_flag;
    for (int item = blockIdx.x; item < s.total; item += gridDim.x) {
        __syncthreads();  // the previous item's LDS use is over
        const int pair = item / S, split = item % S;
        const int b = pair / Hkv, g = pair % Hkv;
        int L = s.gate.seqlens[b];
        L = L < 0 ? 0 : L;
        int nc = L / s.gate.block_size;
        nc = nc > nb_max ? nb_max : nc;
        nc = __builtin_amdgcn_readfirstlane(nc);
        // This split's gate rows; the last split also writes -inf past the complete blocks.
        const int jb = (int)((int64_t)split * nc / S);
        const int je = split == S - 1 ? nb_max : (int)((int64_t)(split + 1) * nc / S);
        gate_rows_item<D, DeviceMem, G>(s.gate, pair, jb, je, sm.gate);
        signal_done(gate_done + pair);
        wait_for(gate_done + pair, S, status);
        // The pair's selection, from its complete scores.
        load_keys(s.gate.scores + (int64_t)pair * nb_max, nc, keys);
        block_select_prepare<256>(sm.sel);
        __syncthreads();  // keys complete
        int32_t *kept = reinterpret_cast<int32_t *>(keys);
        int32_t *out = split == 0 ? const_cast<int32_t *>(s.dec.block_idx) + (int64_t)pair * s.k_max : nullptr;
        const int k = block_select_keys<256, DeviceMem, 2>(keys, nc, SelectPolicy{0, 1, 1, 0.f}, s.k_max, out,
                                                        kept, sm.sel);
        if (split == 0 && threadIdx.x == 0) DeviceMem::sti(const_cast<int32_t *>(s.dec.n_sel) + pair, k);
        __syncthreads();  // kept ids complete; the selection's LDS is free for the decode tiles
        decode_split_item<D, BS, G, DeviceMem, false, false, true>(s.dec, split, g, b, sm.dec, nullptr, kept, k);
        // The pair's last split to finish merges the S partial results.
        if (S > 1 && signal_done_last(dec_done + pair, S, &s_flag)) {
            for (int h = 0; h < G; ++h)
                decode_merge_row<D, DeviceMem>(s.dec.part_o, s.dec.part_ml, S, (int64_t)b * s.dec.Hq + g * G + h,
                                               s.dec.out, s.dec.out_dtype, s.dec.lse, sm.merge);
        }
    }
    // The last workgroup out clears the counters (not the status word) for the next launch.
    __shared__ int s_last;
    __syncthreads();
    if (threadIdx.x == 0)
        s_last = __hip_atomic_fetch_add(ctl + kCtlFinished, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (int)gridDim.x - 1;
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(s_last)) {
        for (int i = threadIdx.x; i < 2 * s.pairs; i += blockDim.x)
            __hip_atomic_store(gate_done + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (threadIdx.x == 0) __hip_atomic_store(ctl + kCtlFinished, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int D, int BS, int G>
static int launch_step(const StepArgs &s, size_t sel_lds_bytes, hipStream_t stream) {
    auto kernel = decode_step_kernel<D, BS, G>;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, sel_lds_bytes) != hipSuccess || per_cu < 1)
        per_cu = 1;
    // A multiple of S (a pair's S items share a round) that is at least S.
    const int S = s.dec.num_splits;
    int grid = device_cu_count() * per_cu;
    grid = grid < s.total ? grid : s.total;
    grid = grid / S * S;
    grid = grid < S ? S : grid;
    kernel<<<dim3(grid), 256, sel_lds_bytes, stream>>>(s);
    return launch_status();
}

template <int D, int BS>
static int step_dispatch_group(const StepArgs &s, size_t lds, int G, hipStream_t stream) {
    switch (G) {
        case 1: return launch_step<D, BS, 1>(s, lds, stream);
        case 2: return launch_step<D, BS, 2>(s, lds, stream);
        case 4: return launch_step<D, BS, 4>(s, lds, stream);
        case 8: return launch_step<D, BS, 8>(s, lds, stream);
    }
    return SEER_ERR_UNSUPPORTED;
}

static size_t step_ctl_bytes(int pairs) { return ((size_t)(kCtlWords + 2 * pairs) * sizeof(int) + 255) / 256 * 256; }

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
    const int S = seer_sparse_decode_num_splits(B, Hkv, k_max, block_size, num_splits);
    if (S > 128 || (int64_t)pairs * (S + 8) > 0x7fffffff / 8) return SEER_ERR_INVALID_ARG;
    if (workspace_bytes < seer_decode_step_workspace_size(B, Hq, Hkv, d, k_max, block_size, S))
        return SEER_ERR_WORKSPACE;

    StepArgs s;
    s.gate = GateArgs{q, sq_b, sq_h, wq, wk, dg, G, Hkv, gate_scale, kpool, nb_max, seqlens, block_size, scores};
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
    s.pairs = pairs;
    s.k_max = k_max;
    s.ctl = reinterpret_cast<int *>(ws);
    s.total = pairs * S;
    const size_t lds = (size_t)nb_max * sizeof(uint32_t);
    if (d == 128)
        return block_size == 128 ? step_dispatch_group<128, 128>(s, lds, G, stream)
                                 : step_dispatch_group<128, 64>(s, lds, G, stream);
    return block_size == 128 ? step_dispatch_group<64, 128>(s, lds, G, stream)
                             : step_dispatch_group<64, 64>(s, lds, G, stream);
}

extern "C" int seer_decode_step_status(const void *workspace, int *status, hipStream_t stream) {
    if (!workspace || !status) return SEER_ERR_INVALID_ARG;
    if (hipMemcpyAsync(status, static_cast<const int *>(workspace) + kCtlStatus, sizeof(int), hipMemcpyDeviceToHost,
                       stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return SEER_ERR_LAUNCH;
    return SEER_OK;
}
