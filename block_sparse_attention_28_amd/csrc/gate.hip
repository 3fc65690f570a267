// gate.hip -- gate scores of one decode step.
//
// Operation: the SeerAttention gate ("SeerAttention: Learning Intrinsic
// Sparse Attention in Your LLMs", abstract v1) projects the pooled query and
// the pooled keys through learnable linear layers and multiplies them into
// block scores.  SeerAttention-R (abstract) removes the query pooling for
// decoding, so the current query row itself is projected.  With one shared
// selection per KV head, the block score is the mean of the group's query-head
// scores; because every step is linear,
//     mean_h (Wq q_h) . (Wk kp_j) = (Wk^T Wq qbar) . kp_j ,   qbar = mean_h q_h,
// so a tiny kernel forms u = gate_scale * Wk^T (Wq qbar) once per (b, g) and
// the bandwidth-bound kernel streams the fp32 pooled keys once:
//     score_j = u . kp_j.
#include "seer_device.hpp"
#include "seer_host.hpp"

namespace seer {

// u[b][g][:] = gate_scale * Wk[g]^T (Wq[g] qbar).  One workgroup per (g, b).
template <int D>
__global__ __launch_bounds__(256) void gate_u_kernel(const uint16_t *q, int64_t sq_b, int64_t sq_h,
                                                     const uint16_t *wq, const uint16_t *wk, int dg, int G, int Hkv,
                                                     float gate_scale, float *u) {
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    __shared__ float qbar[D];
    __shared__ float a_s[256];
    if (tid < D) {
        const uint16_t *qg = q + b * sq_b + (int64_t)(g * G) * sq_h + tid;
        float s = 0.f;
        for (int h = 0; h < G; ++h) s += __uint_as_float((uint32_t)qg[h * sq_h] << 16);
        qbar[tid] = s / (float)G;
    }
    __syncthreads();
    const uint16_t *wqg = wq + (int64_t)g * dg * D;
    for (int rr = wave; rr < dg; rr += 4) {
        float s = 0.f;
#pragma unroll
        for (int e = lane; e < D; e += 64) s = fmaf(__uint_as_float((uint32_t)wqg[(int64_t)rr * D + e] << 16), qbar[e], s);
        s = wave_sum(s);
        if (lane == 0) a_s[rr] = s;
    }
    __syncthreads();
    if (tid < D) {
        const uint16_t *wkg = wk + (int64_t)g * dg * D + tid;
        float s = 0.f;
        for (int rr = 0; rr < dg; ++rr) s = fmaf(__uint_as_float((uint32_t)wkg[(int64_t)rr * D] << 16), a_s[rr], s);
        u[((int64_t)b * Hkv + g) * D + tid] = gate_scale * s;
    }
}

// scores[b][g][j] = u[b][g] . kpool[b][g][j] for j < nc_b, -inf for nc_b <= j < nb_max.
// LPR lanes per pooled-key row (16 bytes = 4 floats each); RPB rows per workgroup.
template <int D>
struct GateScoreCfg {
    static constexpr int LPR = D / 4;           // 32 (d=128) or 16 (d=64)
    static constexpr int ROWS = 256 / LPR;      // rows per workgroup-wide load
    static constexpr int ITER = 8;              // loads in flight per thread
    static constexpr int RPB = ROWS * ITER;     // rows per workgroup
};

template <int D>
__global__ __launch_bounds__(256) void gate_scores_kernel(const float *kpool, int nb_max, const int32_t *seqlens,
                                                          int Hkv, int block_size, const float *u, float *scores) {
    using C = GateScoreCfg<D>;
    const int pair = blockIdx.y;  // b * Hkv + g
    const int b = pair / Hkv;
    const int tid = threadIdx.x, lr = tid / C::LPR, lc = tid % C::LPR;
    int L = seqlens[b];
    L = L < 0 ? 0 : L;
    int nc = L / block_size;
    nc = nc > nb_max ? nb_max : nc;
    const int j0 = blockIdx.x * C::RPB;
    const float4 uu = reinterpret_cast<const float4 *>(u + (int64_t)pair * D)[lc];
    const float *kp = kpool + (int64_t)pair * nb_max * D;
    float4 x[C::ITER];
#pragma unroll
    for (int it = 0; it < C::ITER; ++it) {
        const int j = j0 + lr + it * C::ROWS;
        x[it] = j < nc ? reinterpret_cast<const float4 *>(kp + (int64_t)j * D)[lc] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int it = 0; it < C::ITER; ++it) {
        const int j = j0 + lr + it * C::ROWS;
        float s = uu.x * x[it].x;
        s = fmaf(uu.y, x[it].y, s);
        s = fmaf(uu.z, x[it].z, s);
        s = fmaf(uu.w, x[it].w, s);
        s = group_sum<16>(s);
        if constexpr (C::LPR == 32) s = sum_xor16(s);
        if (lc == 0 && j < nb_max) scores[(int64_t)pair * nb_max + j] = j < nc ? s : -INFINITY;
    }
}

}  // namespace seer

using namespace seer;

extern "C" size_t seer_gate_workspace_size(int B, int Hkv, int d) {
    if (B <= 0 || Hkv <= 0 || d <= 0) return 0;
    return (size_t)B * Hkv * d * sizeof(float);
}

extern "C" int seer_gate_scores(const seer_bf16 *q, int64_t sq_b, int64_t sq_h, const seer_bf16 *wq,
                                const seer_bf16 *wk, int dg, const float *kpool, int nb_max, const int32_t *seqlens,
                                int B, int Hq, int Hkv, int d, int block_size, float gate_scale, float *scores,
                                void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!q || !wq || !wk || !seqlens || !scores) return SEER_ERR_INVALID_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || nb_max < 0 || block_size <= 0 || dg < 1 || dg > 256 ||
        sq_h < 0 || sq_b < 0 || !(gate_scale == gate_scale))
        return SEER_ERR_INVALID_ARG;
    if (nb_max > 0 && (!kpool || !aligned16(kpool))) return SEER_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return SEER_ERR_UNSUPPORTED;
    const size_t need = seer_gate_workspace_size(B, Hkv, d);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return SEER_ERR_WORKSPACE;
    if (Hkv > 65535 || B > 65535 || (int64_t)B * Hkv > 65535) return SEER_ERR_INVALID_ARG;
    float *u = static_cast<float *>(workspace);
    const int G = Hq / Hkv;
    if (d == 128)
        gate_u_kernel<128><<<dim3(Hkv, B), 256, 0, stream>>>(q, sq_b, sq_h, wq, wk, dg, G, Hkv, gate_scale, u);
    else
        gate_u_kernel<64><<<dim3(Hkv, B), 256, 0, stream>>>(q, sq_b, sq_h, wq, wk, dg, G, Hkv, gate_scale, u);
    int st = launch_status();
    if (st != SEER_OK || nb_max == 0) return st;
    if (d == 128) {
        dim3 grid((nb_max + GateScoreCfg<128>::RPB - 1) / GateScoreCfg<128>::RPB, B * Hkv);
        gate_scores_kernel<128><<<grid, 256, 0, stream>>>(kpool, nb_max, seqlens, Hkv, block_size, u, scores);
    } else {
        dim3 grid((nb_max + GateScoreCfg<64>::RPB - 1) / GateScoreCfg<64>::RPB, B * Hkv);
        gate_scores_kernel<64><<<grid, 256, 0, stream>>>(kpool, nb_max, seqlens, Hkv, block_size, u, scores);
    }
    return launch_status();
}
