/*
 * seer_probe.h -- measurement probes used by the benchmark (libseer_probe.so).
 * They are not part of the attention method; they measure two ceilings of the
 * part the method's kernels run on.  All pointers are device pointers; every
 * call only enqueues on `stream` and returns 0, -1 (bad argument) or -4
 * (launch failure).
 */
#ifndef SEER_PROBE_H
#define SEER_PROBE_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core rate: `workgroups` x 256 threads, each wave issuing `iters` x 16
 * independent v_mfma_f32_16x16x32_bf16 (shape 16: 16384 flops each) or
 * `iters` x 8 v_mfma_f32_32x32x16_bf16 (shape 32: 32768 flops each) on register
 * operands.  sink: float [workgroups * 256], written once per thread. */
int seer_probe_mfma_bf16(int shape, float *sink, int workgroups, int iters, hipStream_t stream);

/* Read ceiling of the sparse decode's access pattern: for every (b, KV head),
 * the first `nsel` block ids of block_idx [B][Hkv][k_max] name bf16 K and V
 * blocks of block_size rows x 128 dims ([B][Hkv][kv_capacity][128], strides
 * skv_b, skv_h, contiguous rows), streamed into LDS exactly as the decode loads
 * them, over num_splits workgroups per (b, KV head), with no arithmetic.
 * sink: uint32 [B * Hkv * num_splits]. */
int seer_probe_gather_kv(const uint16_t *k, const uint16_t *v, int64_t skv_b, int64_t skv_h, int kv_capacity,
                         const int32_t *block_idx, int k_max, int nsel, int B, int Hkv, int block_size,
                         int num_splits, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SEER_PROBE_H */
