// select.hip -- token-budget top-k block selection.
//
// Operation ("SeerAttention-R: Sparse Attention Adaptation for Long
// Reasoning", abstract: a fixed token budget at 64/128-token block
// granularity): per (sequence, KV head) keep k = min(budget / bs, nc) complete
// blocks with the largest gate scores, equal scores ordered by the lower block
// id, and emit the kept ids in ascending order (so decoding reads memory
// forward).
//
// One workgroup per (b, head).  Scores become order-preserving 32-bit keys
// held in LDS; an 8-bit-digit radix select (four histogram passes from the
// most significant digit) finds the k-th largest key T exactly and how many
// keys equal to T must be taken; a last pass keeps keys > T plus the first
// `need` keys == T in id order, and a block-wide prefix sum places each kept
// id at its ascending position.  All decisions are integer comparisons of the
// fp32 score bits.
#include "seer_device.hpp"
#include "seer_host.hpp"

namespace seer {

constexpr int kSelThreads = 256;
constexpr int kSelMaxBlocks = 16384;

__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (s == 0.0f) u = 0u;  // +0 and -0 compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 256 threads (Hillis-Steele in LDS).
__device__ __forceinline__ int block_inclusive_scan(int v, int *buf) {
    const int tid = threadIdx.x;
    buf[tid] = v;
    __syncthreads();
#pragma unroll
    for (int off = 1; off < kSelThreads; off <<= 1) {
        const int add = tid >= off ? buf[tid - off] : 0;
        __syncthreads();
        buf[tid] += add;
        __syncthreads();
    }
    const int r = buf[tid];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kSelThreads) void select_blocks_kernel(const float *scores, const int32_t *seqlens,
                                                                    int H, int nb_max, int block_size, int k_max,
                                                                    int32_t *block_idx, int32_t *n_sel) {
    extern __shared__ uint32_t keys[];  // [nb_max]
    __shared__ int hist[256];
    __shared__ int scan_buf[kSelThreads];
    __shared__ int s_digit, s_need;

    const int pair = blockIdx.x;  // b * H + h
    const int b = pair / H, tid = threadIdx.x;
    int L = seqlens[b];
    L = L < 0 ? 0 : L;
    int nc = L / block_size;
    nc = nc > nb_max ? nb_max : nc;
    const int k = k_max < nc ? k_max : nc;
    int32_t *out = block_idx + (int64_t)pair * k_max;

    if (k == nc || k == 0) {  // every complete block, or none, is kept
        for (int i = tid; i < k_max; i += kSelThreads) out[i] = i < k ? i : -1;
        if (tid == 0) n_sel[pair] = k;
        return;
    }
    const float *sc = scores + (int64_t)pair * nb_max;
    for (int j = tid; j < nc; j += kSelThreads) keys[j] = order_key(sc[j]);

    uint32_t prefix = 0;
    int need = k;  // keys still to take at or below the current prefix
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        hist[tid] = 0;
        __syncthreads();
        for (int j = tid; j < nc; j += kSelThreads) {
            const uint32_t key = keys[j];
            const bool match = pass == 0 || (key >> (shift + 8)) == (prefix >> (shift + 8));
            if (match) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
        __syncthreads();
        // thread t looks at digit 255 - t; cumulative count from the top digit down
        const int cnt = hist[255 - tid];
        const int incl = block_inclusive_scan(cnt, scan_buf);
        if (incl >= need && incl - cnt < need) {
            s_digit = 255 - tid;
            s_need = need - (incl - cnt);
        }
        __syncthreads();
        prefix |= (uint32_t)s_digit << shift;
        need = s_need;
        __syncthreads();
    }
    const uint32_t T = prefix;

    // Contiguous id range per thread so that prefix sums follow id order.
    const int per = (nc + kSelThreads - 1) / kSelThreads;
    const int j_lo = tid * per, j_hi = (j_lo + per) < nc ? (j_lo + per) : nc;
    int eq_local = 0;
    for (int j = j_lo; j < j_hi; ++j) eq_local += keys[j] == T;
    const int eq_before = block_inclusive_scan(eq_local, scan_buf) - eq_local;
    int take_local = 0, eq_seen = eq_before;
    for (int j = j_lo; j < j_hi; ++j) {
        const uint32_t key = keys[j];
        if (key > T) ++take_local;
        else if (key == T) take_local += (eq_seen++ < need);
    }
    int pos = block_inclusive_scan(take_local, scan_buf) - take_local;
    eq_seen = eq_before;
    for (int j = j_lo; j < j_hi; ++j) {
        const uint32_t key = keys[j];
        bool take = key > T;
        if (key == T) take = eq_seen++ < need;
        if (take && pos < k) out[pos++] = j;
    }
    for (int i = k + tid; i < k_max; i += kSelThreads) out[i] = -1;
    if (tid == 0) n_sel[pair] = k;
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
    if ((int64_t)B * H > 0x7fffffffLL) return SEER_ERR_INVALID_ARG;
    const size_t shmem = (size_t)(nb_max > 0 ? nb_max : 1) * sizeof(uint32_t);
    select_blocks_kernel<<<dim3(B * H), kSelThreads, shmem, stream>>>(scores, seqlens, H, nb_max, block_size, k_max,
                                                                      block_idx, n_sel);
    return launch_status();
}
