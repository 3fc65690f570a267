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
// A work item owns a range of pooled-key rows of one (b, g): it issues the
// loads of the query rows and gate weights (L2-resident), then a batch of RPB
// pooled-key rows (16 bytes per lane, ITER rows in flight per thread), forms u
// while the pooled rows arrive, then finishes the dot products with 32-lane
// DPP/permlane reductions, batch after batch.
#pragma once

#include "seer_device.hpp"

namespace seer {

template <int D, int NT = 256>
struct GateCfg {
    static constexpr int LPR = D / 4;        // lanes per pooled-key row (4 floats each)
    static constexpr int ROWS = NT / LPR;    // rows per workgroup-wide load
    static constexpr int ITER = NT >= 1024 ? 8 : 16;  // row loads in flight per thread
    static constexpr int RPB = ROWS * ITER;  // rows per batch: 128 (d 128) at 256 threads, 256 at 1024
    static constexpr int CH = D / 8;         // 16-byte bf16 chunks per weight row: 16 or 8
    static constexpr int RG = 256 / CH;      // weight-row groups of the first 256 threads: 16 or 32
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

// The gate vector u = gate_scale * Wk^T (Wq qbar) of (b, g) in one fixed
// order: "thread" t < 256 owns the 16-byte column chunk t % CH of weight rows
// t / CH + RG i; it forms a[r] = Wq[r] . qbar for its Wq rows, then its share
// u_part[t / CH] of Wk^T a over its Wk rows.  issue() starts the loads of the
// query rows and of the first Wq and Wk rows, through buffer descriptors whose
// ranges end at the last valid row, so heads >= G and weight rows >= dg read as
// zero and no branch separates the loads.  finish() leaves u in sm.u; every
// thread of the workgroup calls it (it holds barriers).  With SPLIT (workgroups
// of 512 threads or more) thread 256 + t holds t's Wk rows and does its Wk
// share, so every weight row is in flight from the start without one thread
// holding both; the arithmetic, and hence u, is the same bit for bit.
template <int D, int QB, bool SPLIT = false>
struct GateU {
    using C = GateCfg<D>;
    static constexpr int WB = 8;  // weight rows per thread in flight
    uint4 qw[QB], wv[WB], wkv[SPLIT ? 1 : WB];  // wv: Wq rows (threads < 256), or Wk rows (SPLIT, 256..511)

    __device__ __forceinline__ void issue(const GateArgs &ga, int b, int g) {
        const int tid = threadIdx.x, t = tid & 255, c = t % C::CH, rg = t / C::CH;
        const uint16_t *qg = ga.q + b * ga.sq_b + (int64_t)(g * ga.G) * ga.sq_h;
        const auto qrs = buffer_rsrc(qg, (uint32_t)(((int64_t)(ga.G - 1) * ga.sq_h + D) * 2));
        const auto wqrs = buffer_rsrc(ga.wq + (int64_t)g * ga.dg * D, (uint32_t)(ga.dg * D * 2));
        const auto wkrs = buffer_rsrc(ga.wk + (int64_t)g * ga.dg * D, (uint32_t)(ga.dg * D * 2));
        auto wrow = [&](int r) { return (uint32_t)(r * D * 2 + c * 16); };
        if (tid < 256) {
#pragma unroll
            for (int h = 0; h < QB; ++h) qw[h] = buf_ld16(qrs, (uint32_t)(h * ga.sq_h * 2) + c * 16, 0);
#pragma unroll
            for (int i = 0; i < WB; ++i) wv[i] = buf_ld16(wqrs, wrow(rg + i * C::RG), 0);
            if constexpr (!SPLIT) {
#pragma unroll
                for (int i = 0; i < WB; ++i) wkv[i] = buf_ld16(wkrs, wrow(rg + i * C::RG), 0);
            }
        } else if (SPLIT && tid < 512) {
#pragma unroll
            for (int i = 0; i < WB; ++i) wv[i] = buf_ld16(wkrs, wrow(rg + i * C::RG), 0);
        }
    }

    __device__ __forceinline__ void finish(const GateArgs &ga, int b, int g, GateSmem<D> &sm) {
        const int tid = threadIdx.x, t = tid & 255, c = t % C::CH, rg = t / C::CH;
        const int dg = ga.dg, G = ga.G;
        const uint16_t *qg = ga.q + b * ga.sq_b + (int64_t)(g * G) * ga.sq_h;
        const auto wqrs = buffer_rsrc(ga.wq + (int64_t)g * dg * D, (uint32_t)(dg * D * 2));
        const auto wkrs = buffer_rsrc(ga.wk + (int64_t)g * dg * D, (uint32_t)(dg * D * 2));
        auto wrow = [&](int r) { return (uint32_t)(r * D * 2 + c * 16); };
        if (tid < 256) {  // a[r] = Wq[r] . qbar, qbar the mean of the group's query heads
            float qb[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int h = 0; h < QB; ++h) {
                if (h < G) {
                    float f[8];
                    unpack8(qw[h], f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) qb[e] += f[e];
                }
            }
            for (int h = QB; h < G; ++h) {  // groups wider than QB heads
                float f[8];
                unpack8(*reinterpret_cast<const uint4 *>(qg + h * ga.sq_h + c * 8), f);
#pragma unroll
                for (int e = 0; e < 8; ++e) qb[e] += f[e];
            }
            const float inv_g = 1.0f / (float)G;
#pragma unroll
            for (int e = 0; e < 8; ++e) qb[e] *= inv_g;
            for (int r0 = 0; r0 < dg; r0 += WB * C::RG) {
                if (r0 > 0) {
#pragma unroll
                    for (int i = 0; i < WB; ++i) wv[i] = buf_ld16(wqrs, wrow(r0 + rg + i * C::RG), 0);
                }
#pragma unroll
                for (int i = 0; i < WB; ++i) {
                    const int r = r0 + rg + i * C::RG;
                    float f[8];
                    unpack8(wv[i], f);
                    float s = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) s = fmaf(f[e], qb[e], s);
                    s = group_sum<C::CH>(s);  // all CH lanes of a row group share r
                    if (c == 0 && r < dg) sm.a[r] = s;
                }
            }
        }
        __syncthreads();
        // u_part[rg] = sum over t's Wk rows of a[r] Wk[r], by thread t or (SPLIT) 256 + t
        if (SPLIT ? (tid >= 256 && tid < 512) : tid < 256) {
            uint4 *wk_rows = SPLIT ? wv : wkv;
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int r0 = 0; r0 < dg; r0 += WB * C::RG) {
                if (r0 > 0) {
#pragma unroll
                    for (int i = 0; i < WB; ++i) wk_rows[i] = buf_ld16(wkrs, wrow(r0 + rg + i * C::RG), 0);
                }
#pragma unroll
                for (int i = 0; i < WB; ++i) {
                    const int r = r0 + rg + i * C::RG;
                    float f[8];
                    unpack8(wk_rows[i], f);
                    const float ar = r < dg ? sm.a[r] : 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] = fmaf(ar, f[e], acc[e]);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.u_part[rg][c * 8 + e] = acc[e];
        }
        __syncthreads();
        if (tid < D) {
            float s = 0.f;
#pragma unroll
            for (int r = 0; r < C::RG; ++r) s += sm.u_part[r][tid];
            sm.u[tid] = s * ga.gate_scale;
        }
        __syncthreads();
    }
};

// Rows [jb, je) of the scores of pair = b * Hkv + g (je <= nb_max): u . kp_j
// for the complete blocks among them, -inf for the rest.  Every thread of the
// NT-thread workgroup calls it.  QB: query rows loaded up front (at least
// min(G, 8) keeps every row of a group of up to 8 in flight with the weights;
// rows past QB are loaded when used).
template <int D, class Mem, int QB = 8, int NT = 256>
__device__ __forceinline__ void gate_rows_item(const GateArgs &ga, int pair, int jb, int je, GateSmem<D> &sm) {
    using C = GateCfg<D, NT>;
    const int nb_max = ga.nb_max;
    const int b = pair / ga.Hkv, g = pair % ga.Hkv;
    const int tid = threadIdx.x, lr = tid / C::LPR, lc = tid % C::LPR;
    int L = ga.seqlens[b];
    L = L < 0 ? 0 : L;
    int nc = L / ga.block_size;
    nc = nc > nb_max ? nb_max : nc;
    const int jv = je < nc ? je : nc;  // rows [jb, jv) are complete blocks
    float *srow = ga.scores + (int64_t)pair * nb_max;
    for (int j = (jb > jv ? jb : jv) + tid; j < je; j += NT) Mem::stf(srow + j, -INFINITY);
    if (jb >= jv) return;  // nothing complete here

    // 1. Loads in the order they are used: the query rows and the first Wq and
    // Wk rows (L2-resident), then this item's pooled-key rows (rows past jv read
    // as zero).  A barrier between the two puts every wave's weight requests
    // ahead of the pooled-key stream, so u is formed while the pooled rows are
    // still arriving.
    GateU<D, QB, (NT >= 512)> gu;
    gu.issue(ga, b, g);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const auto kprs = buffer_rsrc(ga.kpool + (int64_t)pair * nb_max * D, (uint32_t)jv * D * 4);
    float4 x[C::ITER];
#pragma unroll
    for (int it = 0; it < C::ITER; ++it)
        x[it] = as_float4(buf_ld16_nt(kprs, (uint32_t)((jb + lr + it * C::ROWS) * D * 4 + lc * 16), 0));
    __builtin_amdgcn_sched_barrier(0);

    // 2. u
    gu.finish(ga, b, g, sm);

    // 3. score_j = u . kp_j, RPB rows at a time.
    const float4 uu = reinterpret_cast<const float4 *>(sm.u)[lc];
    for (int j0 = jb;;) {
#pragma unroll
        for (int it = 0; it < C::ITER; ++it) {
            const int j = j0 + lr + it * C::ROWS;
            float s = uu.x * x[it].x;
            s = fmaf(uu.y, x[it].y, s);
            s = fmaf(uu.z, x[it].z, s);
            s = fmaf(uu.w, x[it].w, s);
            s = group_sum<16>(s);
            if constexpr (C::LPR == 32) s = sum_xor16(s);
            if (lc == 0 && j < jv) Mem::stf(srow + j, s);
        }
        j0 += C::RPB;
        if (j0 >= jv) break;
#pragma unroll
        for (int it = 0; it < C::ITER; ++it)
            x[it] = as_float4(buf_ld16_nt(kprs, (uint32_t)((j0 + lr + it * C::ROWS) * D * 4 + lc * 16), 0));
    }
}

}  // namespace seer
