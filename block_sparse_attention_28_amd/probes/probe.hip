// probe.hip -- measurement probes for the benchmark (not part of the method).
//
// Two ceilings the benchmark reports beside its roofline fractions:
//   * the bf16 matrix-core rate this part sustains: every wave of a full grid
//     issues independent v_mfma_f32_16x16x32_bf16 (or 32x32x16) on register
//     operands, so nothing but the matrix cores bounds it;
//   * the rate at which the sparse decode's access pattern can be read at
//     all: the kept K and V blocks of every (sequence, KV head) streamed into
//     LDS with the decode's own loads (LDS-direct, non-temporal, a quarter of
//     a block per wave), with no arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "seer_probe.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kChains = 16;  // independent accumulators per wave

__global__ __launch_bounds__(256) void mfma_16x16x32_kernel(float *sink, int iters) {
    const int t = threadIdx.x;
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(1.0f + 0.001f * (float)((t + i) & 7));
        b[i] = (__bf16)(0.5f - 0.001f * (float)((t * 3 + i) & 7));
    }
    f32x4_t acc[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    sink[blockIdx.x * blockDim.x + t] = s;
}

__global__ __launch_bounds__(256) void mfma_32x32x16_kernel(float *sink, int iters) {
    const int t = threadIdx.x;
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(1.0f + 0.001f * (float)((t + i) & 7));
        b[i] = (__bf16)(0.5f - 0.001f * (float)((t * 3 + i) & 7));
    }
    f32x16_t acc[kChains / 2];
#pragma unroll
    for (int j = 0; j < kChains / 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains / 2; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kChains / 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    sink[blockIdx.x * blockDim.x + t] = s;
}

// One workgroup per (split, KV head, sequence), as the decode: the kept blocks
// of the pair cut into 32-token slices, divided over the splits, and dealt
// round-robin to the waves.
template <int BS>
__global__ __launch_bounds__(256) void gather_kv_kernel(const uint16_t *k, const uint16_t *v, int64_t skv_b,
                                                        int64_t skv_h, int kv_capacity, const int32_t *block_idx,
                                                        int k_max, int nsel, int num_splits, int Hkv,
                                                        uint32_t *sink) {
    constexpr int D = 128, TPW = 32, SPB = BS / TPW, NDMA = TPW / 4;  // 4 rows of 256 B per 1 KiB load
    __shared__ __attribute__((aligned(16))) uint16_t kt[4][TPW * D], vt[4][TPW * D];
    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint16_t *kb = k + b * skv_b + g * skv_h, *vb = v + b * skv_b + g * skv_h;
    const uint32_t region = (uint32_t)((int64_t)kv_capacity * D * 2);
    const auto krs = __builtin_amdgcn_make_buffer_rsrc((void *)kb, 0, region, 0x00020000);
    const auto vrs = __builtin_amdgcn_make_buffer_rsrc((void *)vb, 0, region, 0x00020000);
    const int32_t *sel = block_idx + (int64_t)(b * Hkv + g) * k_max;
    const int64_t ns = (int64_t)nsel * SPB;
    const int i0 = (int)((split * ns) / num_splits), i1 = (int)(((split + 1) * ns) / num_splits);
    const int r0 = __builtin_amdgcn_readfirstlane((i0 - wave + 3) / 4);
    const int r1 = __builtin_amdgcn_readfirstlane((i1 - wave + 3) / 4);
    const uint32_t lane_off = (uint32_t)(((lane / 16) * D + (lane % 16) * 8) * 2);
    char *kt_w = reinterpret_cast<char *>(kt[wave]), *vt_w = reinterpret_cast<char *>(vt[wave]);
    const int nb = kv_capacity / BS;
    for (int r = r0; r < r1; ++r) {
        const int sl = 4 * r + wave;  // < ns, so its block sl / SPB < nsel
        int blk = __builtin_amdgcn_readfirstlane(sel[sl / SPB]);
        blk = blk < 0 ? 0 : (blk >= nb ? nb - 1 : blk);  // stays inside the cache
        const uint32_t soff = (uint32_t)(blk * BS + (sl % SPB) * TPW) * D * 2u;
#pragma unroll
        for (int q = 0; q < NDMA; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void *)(kt_w + q * 1024), 16,
                                                     (int)(lane_off + q * 1024), (int)soff, 0, 2);
#pragma unroll
        for (int q = 0; q < NDMA; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void *)(vt_w + q * 1024), 16,
                                                     (int)(lane_off + q * 1024), (int)soff, 0, 2);
        __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    __syncthreads();
    if (threadIdx.x == 0) sink[(b * Hkv + g) * num_splits + split] = reinterpret_cast<uint32_t *>(kt[0])[0];
}

int status() { return hipGetLastError() == hipSuccess ? 0 : -4; }

}  // namespace

extern "C" int seer_probe_mfma_bf16(int shape, float *sink, int workgroups, int iters, hipStream_t stream) {
    if (!sink || workgroups <= 0 || iters <= 0 || (shape != 16 && shape != 32)) return -1;
    if (shape == 16)
        mfma_16x16x32_kernel<<<dim3(workgroups), 256, 0, stream>>>(sink, iters);
    else
        mfma_32x32x16_kernel<<<dim3(workgroups), 256, 0, stream>>>(sink, iters);
    return status();
}

extern "C" int seer_probe_gather_kv(const uint16_t *k, const uint16_t *v, int64_t skv_b, int64_t skv_h,
                                    int kv_capacity, const int32_t *block_idx, int k_max, int nsel, int B, int Hkv,
                                    int block_size, int num_splits, uint32_t *sink, hipStream_t stream) {
    if (!k || !v || !block_idx || !sink || B <= 0 || Hkv <= 0 || nsel < 0 || nsel > k_max || num_splits <= 0 ||
        (block_size != 64 && block_size != 128) || kv_capacity < block_size ||
        (int64_t)kv_capacity * 256 > 0x7fffffffLL)
        return -1;
    const dim3 grid(num_splits, Hkv, B);
    if (block_size == 128)
        gather_kv_kernel<128><<<grid, 256, 0, stream>>>(k, v, skv_b, skv_h, kv_capacity, block_idx, k_max, nsel,
                                                         num_splits, Hkv, sink);
    else
        gather_kv_kernel<64><<<grid, 256, 0, stream>>>(k, v, skv_b, skv_h, kv_capacity, block_idx, k_max, nsel,
                                                        num_splits, Hkv, sink);
    return status();
}
