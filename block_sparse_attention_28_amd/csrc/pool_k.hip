// pool_k.hip -- pooled-key cache update.
//
// Operation ("SeerAttention: Learning Intrinsic Sparse Attention in Your
// LLMs", abstract v1): the gate pools K along the sequence, one vector per
// block; here the pooling is the mean over the block's tokens, stored in fp32
// so the gate's fp32 scores rank blocks as an fp64 evaluation would.  Decoding
// keeps this pooling (SeerAttention-R abstract), so the cache grows by one row
// whenever a sequence completes a block.
//
// One workgroup per (listed block, KV head): 256 threads read the bs x d bf16
// block as 16-byte chunks (a 256-byte row per 16 threads, fully coalesced),
// accumulate in fp32 and reduce the row groups through LDS in a fixed order,
// so the result is bitwise reproducible whichever call pools the block.
#include "seer_device.hpp"
#include "seer_host.hpp"

namespace seer {

template <int D, int BS, class KT>
__global__ __launch_bounds__(256) void pool_k_kernel(const uint16_t *k, int64_t sk_b, int64_t sk_h, int64_t sk_t,
                                                     int B, int Hkv, int kv_capacity, const int32_t *upd_b,
                                                     const int32_t *upd_blk, KT *kpool, int nb_max) {
    constexpr int CH = D / 8, RG = 256 / CH;  // chunks per row, row groups
    const int i = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const int b = upd_b[i], j = upd_blk[i];
    if (b < 0 || b >= B || j < 0 || j >= nb_max || (int64_t)(j + 1) * BS > kv_capacity) return;
    const int c = tid % CH, rg = tid / CH;
    const uint16_t *base = k + b * sk_b + h * sk_h + (int64_t)j * BS * sk_t + c * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // Streaming loads: a block is pooled once, and caching it would only push
    // out lines that other work reuses.
    uint4 rows[BS / RG];
#pragma unroll
    for (int i = 0; i < BS / RG; ++i) {
        const u32x4_t t =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(base + (int64_t)(rg + i * RG) * sk_t));
        rows[i] = make_uint4(t.x, t.y, t.z, t.w);
    }
#pragma unroll
    for (int i = 0; i < BS / RG; ++i) {
        const uint4 w = rows[i];
        acc[0] += bf16lo(w.x); acc[1] += bf16hi(w.x);
        acc[2] += bf16lo(w.y); acc[3] += bf16hi(w.y);
        acc[4] += bf16lo(w.z); acc[5] += bf16hi(w.z);
        acc[6] += bf16lo(w.w); acc[7] += bf16hi(w.w);
    }
    __shared__ float part[RG][D];
#pragma unroll
    for (int e = 0; e < 8; ++e) part[rg][c * 8 + e] = acc[e];
    __syncthreads();
    if (tid < D) {
        float s = 0.f;
#pragma unroll
        for (int g = 0; g < RG; ++g) s += part[g][tid];
        const float mean = s * (1.0f / BS);  // exact scaling: BS is a power of two
        const int64_t at = (((int64_t)b * Hkv + h) * nb_max + j) * D + tid;
        if constexpr (sizeof(KT) == 4)
            kpool[at] = mean;
        else
            kpool[at] = f32_to_bf16(mean);  // the bf16 table: round to nearest even
    }
}

}  // namespace seer

using namespace seer;

extern "C" int seer_pool_k_blocks_ex(const seer_bf16 *k, int64_t sk_b, int64_t sk_h, int64_t sk_t, int B, int Hkv,
                                     int d, int block_size, int kv_capacity, const int32_t *upd_b,
                                     const int32_t *upd_blk, int n_upd, void *kpool, int kpool_dtype, int nb_max,
                                     hipStream_t stream) {
    if (n_upd < 0 || B <= 0 || Hkv <= 0 || nb_max < 0 || kv_capacity < 0) return SEER_ERR_INVALID_ARG;
    if (kpool_dtype != SEER_KPOOL_F32 && kpool_dtype != SEER_KPOOL_BF16) return SEER_ERR_INVALID_ARG;
    if (n_upd == 0) return SEER_OK;
    if (!k || !upd_b || !upd_blk || !kpool || !rows_aligned16(k, sk_t) || sk_h % 8 || sk_b % 8 || sk_t < d ||
        !aligned16(kpool))
        return SEER_ERR_INVALID_ARG;
    if ((d != 64 && d != 128) || (block_size != 64 && block_size != 128)) return SEER_ERR_UNSUPPORTED;
    if (Hkv > 65535) return SEER_ERR_INVALID_ARG;
    dim3 grid(n_upd, Hkv);
    float *kp32 = static_cast<float *>(kpool);
    uint16_t *kp16 = static_cast<uint16_t *>(kpool);
#define SEER_POOL(D_, BS_)                                                                                           \
    do {                                                                                                             \
        if (kpool_dtype == SEER_KPOOL_F32)                                                                           \
            pool_k_kernel<D_, BS_, float><<<grid, 256, 0, stream>>>(k, sk_b, sk_h, sk_t, B, Hkv, kv_capacity, upd_b, \
                                                                    upd_blk, kp32, nb_max);                          \
        else                                                                                                         \
            pool_k_kernel<D_, BS_, uint16_t><<<grid, 256, 0, stream>>>(k, sk_b, sk_h, sk_t, B, Hkv, kv_capacity,     \
                                                                       upd_b, upd_blk, kp16, nb_max);                \
    } while (0)
    if (d == 128) {
        if (block_size == 128) SEER_POOL(128, 128); else SEER_POOL(128, 64);
    } else {
        if (block_size == 128) SEER_POOL(64, 128); else SEER_POOL(64, 64);
    }
#undef SEER_POOL
    return launch_status();
}

extern "C" int seer_pool_k_blocks(const seer_bf16 *k, int64_t sk_b, int64_t sk_h, int64_t sk_t, int B, int Hkv,
                                  int d, int block_size, int kv_capacity, const int32_t *upd_b,
                                  const int32_t *upd_blk, int n_upd, float *kpool, int nb_max, hipStream_t stream) {
    return seer_pool_k_blocks_ex(k, sk_b, sk_h, sk_t, B, Hkv, d, block_size, kv_capacity, upd_b, upd_blk, n_upd,
                                 kpool, SEER_KPOOL_F32, nb_max, stream);
}
