// gate_items.hpp -- device body of the gate scores of one decode step.
//
// Operation: the SeerAttention gate ("SeerAttention: Learning Intrinsic
// Sparse Attention in Your LLMs", abstract v1) projects the pooled query and
// the pooled keys through learnable linear layers and multiplies them into
// block scores.  SeerAttention-R (abstract) removes the query pooling for
// decoding, so the current query row itself is projected.  With one shared
// selection per KV head, the block score is the mean of the group's query-head
// scores; because every step is linear,
//     mean_h (Wq q_h) . (Wk kp_j) = (Wk^T Wq qbar) . kp_j ,   qbar = mean_h q_h,
// so each workgroup forms u = gate_scale * Wk^T (Wq qbar) for its (b, g) and
// then streams fp32 pooled keys once: score_j = u . kp_j.
//
// A work item owns RPB consecutive pooled-key rows of one (b, g):
// it issues all of their loads first (16 bytes per lane, 4 rows in flight per
// thread and per load instruction), computes u from the L2-resident gate
// weights while those loads are in flight, then finishes the dot products
// with 32-lane DPP/permlane reductions.
#pragma once

#include "seer_device.hpp"

namespace seer {

template <int D>
struct GateCfg {
    static constexpr int LPR = D / 4;        // lanes per pooled-key row (4 floats each)
    static constexpr int ROWS = 256 / LPR;   // rows per workgroup-wide load: 8 or 16
    static constexpr int ITER = 16;          // row loads in flight per thread
    static constexpr int RPB = ROWS * ITER;  // rows per workgroup
    static constexpr int CH = D / 8;         // 16-byte bf16 chunks per weight row: 16 or 8
    static constexpr int RG = 256 / CH;      // weight-row groups: 16 or 32
};

__device__ __forceinline__ void unpack8(const uint4 w, float *f) {
    f[0] = bf16lo(w.x); f[1] = bf16hi(w.x); f[2] = bf16lo(w.y); f[3] = bf16hi(w.y);
    f[4] = bf16lo(w.z); f[5] = bf16hi(w.z); f[6] = bf16lo(w.w); f[7] = bf16hi(w.w);
}

struct GateArgs {
    const uint16_t *q;
    int64_t sq_b, sq_h;
    const uint16_t *wq, *wk;
    int dg, G, Hkv;
    float gate_scale;
    const float *kpool;
    int nb_max;
    const int32_t *seqlens;
    int block_size;
    float *scores;
};

template <int D>
struct GateSmem {
    float a[256];
    float u_part[GateCfg<D>::RG][D];
    float u[D];
};

// Rows [chunk * RPB, (chunk + 1) * RPB) of the scores of pair = b * Hkv + g.
// Every thread of the 256-thread workgroup calls it.
template <int D, class Mem>
__device__ __forceinline__ void gate_chunk_item(const GateArgs &ga, int chunk, int pair, GateSmem<D> &sm) {
    const uint16_t *q = ga.q;
    const int64_t sq_b = ga.sq_b, sq_h = ga.sq_h;
    const uint16_t *wq = ga.wq, *wk = ga.wk;
    const int dg = ga.dg, G = ga.G, Hkv = ga.Hkv;
    const float gate_scale = ga.gate_scale;
    const float *kpool = ga.kpool;
    const int nb_max = ga.nb_max, block_size = ga.block_size;
    const int32_t *seqlens = ga.seqlens;
    float *scores = ga.scores;
    auto &a_s = sm.a;
    auto &u_part = sm.u_part;
    auto &u_s = sm.u;
    using C = GateCfg<D>;
    const int b = pair / Hkv, g = pair % Hkv;
    const int tid = threadIdx.x, lr = tid / C::LPR, lc = tid % C::LPR;
    int L = seqlens[b];
    L = L < 0 ? 0 : L;
    int nc = L / block_size;
    nc = nc > nb_max ? nb_max : nc;
    const int j0 = chunk * C::RPB;
    float *srow = scores + (int64_t)pair * nb_max;
    if (j0 >= nc) {  // nothing complete here: only -inf to write
        for (int j = j0 + tid; j < j0 + C::RPB && j < nb_max; j += 256) Mem::stf(srow + j, -INFINITY);
        return;
    }

    // 1. Pooled-key rows of this workgroup, all loads issued up front.
    const float *kp = kpool + (int64_t)pair * nb_max * D;
    float4 x[C::ITER];
#pragma unroll
    for (int it = 0; it < C::ITER; ++it) {
        const int j = j0 + lr + it * C::ROWS;
        x[it] = j < nc ? reinterpret_cast<const float4 *>(kp + (int64_t)j * D)[lc] : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // 2. u = gate_scale * Wk^T (Wq qbar) for (b, g).
    const int c = tid % C::CH, rg = tid / C::CH;
    // Each thread owns the 16-byte column chunk c of weight rows rg, rg + RG, ...,
    // taken 8 rows at a time with all 8 loads issued before any is used.
    constexpr int WB = 8;
    const uint16_t *qg = q + b * sq_b + (int64_t)(g * G) * sq_h + c * 8;
    float qb[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int h0 = 0; h0 < G; h0 += 4) {
        uint4 qw[4];
#pragma unroll
        for (int h = 0; h < 4; ++h)
            qw[h] = h0 + h < G ? *reinterpret_cast<const uint4 *>(qg + (h0 + h) * sq_h) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            float f[8];
            unpack8(qw[h], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) qb[e] += f[e];
        }
    }
    const float inv_g = 1.0f / (float)G;
#pragma unroll
    for (int e = 0; e < 8; ++e) qb[e] *= inv_g;
    const uint16_t *wqg = wq + (int64_t)g * dg * D + c * 8;
    const uint16_t *wkg = wk + (int64_t)g * dg * D + c * 8;
    for (int r0 = 0; r0 < dg; r0 += WB * C::RG) {  // a[r] = Wq[r] . qbar
        uint4 w[WB];
#pragma unroll
        for (int i = 0; i < WB; ++i) {
            const int r = r0 + rg + i * C::RG;
            w[i] = r < dg ? *reinterpret_cast<const uint4 *>(wqg + (int64_t)r * D) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < WB; ++i) {
            const int r = r0 + rg + i * C::RG;
            float f[8];
            unpack8(w[i], f);
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) s = fmaf(f[e], qb[e], s);
            s = group_sum<C::CH>(s);  // all CH lanes of a row group share r
            if (c == 0 && r < dg) a_s[r] = s;
        }
    }
    __syncthreads();
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int r0 = 0; r0 < dg; r0 += WB * C::RG) {  // u += a[r] * Wk[r]
        uint4 w[WB];
#pragma unroll
        for (int i = 0; i < WB; ++i) {
            const int r = r0 + rg + i * C::RG;
            w[i] = r < dg ? *reinterpret_cast<const uint4 *>(wkg + (int64_t)r * D) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < WB; ++i) {
            const int r = r0 + rg + i * C::RG;
            float f[8];
            unpack8(w[i], f);
            const float ar = r < dg ? a_s[r] : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = fmaf(ar, f[e], acc[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) u_part[rg][c * 8 + e] = acc[e];
    __syncthreads();
    if (tid < D) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < C::RG; ++r) s += u_part[r][tid];
        u_s[tid] = s * gate_scale;
    }
    __syncthreads();

    // 3. score_j = u . kp_j
    const float4 uu = reinterpret_cast<const float4 *>(u_s)[lc];
#pragma unroll
    for (int it = 0; it < C::ITER; ++it) {
        const int j = j0 + lr + it * C::ROWS;
        float s = uu.x * x[it].x;
        s = fmaf(uu.y, x[it].y, s);
        s = fmaf(uu.z, x[it].z, s);
        s = fmaf(uu.w, x[it].w, s);
        s = group_sum<16>(s);
        if constexpr (C::LPR == 32) s = sum_xor16(s);
        if (lc == 0 && j < nb_max) Mem::stf(srow + j, j < nc ? s : -INFINITY);
    }
}

}  // namespace seer
