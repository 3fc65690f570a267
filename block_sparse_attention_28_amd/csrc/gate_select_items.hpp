// gate_select_items.hpp -- gate scores and token-budget selection of one
// (b, KV head) by one workgroup.
//
// Same operation as gate_rows_item over all rows of a pair followed by the
// selection (see gate_items.hpp and topk_wave.hpp for the definitions this
// follows), arranged so that the scores never leave the workgroup:
//
//  1. Loads are issued in the order q, Wq, Wk, pooled keys.  The gate vector
//     u = gate_scale * Wk^T (Wq qbar) only needs the first three, so its
//     dependent chain (two small products and three barriers) runs while the
//     pooled-key rows are still arriving.
//  2. score_j = u . kp_j for the complete blocks, written to the scores output
//     and, as order-preserving keys, to LDS.
//  3. The block-wide selection of topk_block.hpp over those LDS keys.
#pragma once

#include "gate_items.hpp"
#include "topk_block.hpp"
#include "topk_wave.hpp"

namespace seer {

// Element type of the pooled-key table: fp32, or bf16 bits (half the bytes).
template <class KT>
struct KRow;
template <>
struct KRow<float> {
    static constexpr int KB = 4, EPL = 4;  // bytes per element, elements per 16-byte lane load
    __device__ static float dot(const float *u, uint4 x) {
        float s = u[0] * __uint_as_float(x.x);
        s = fmaf(u[1], __uint_as_float(x.y), s);
        s = fmaf(u[2], __uint_as_float(x.z), s);
        return fmaf(u[3], __uint_as_float(x.w), s);
    }
};
template <>
struct KRow<uint16_t> {
    static constexpr int KB = 2, EPL = 8;
    __device__ static float dot(const float *u, uint4 x) {
        float s = u[0] * bf16lo(x.x);
        s = fmaf(u[1], bf16hi(x.x), s);
        s = fmaf(u[2], bf16lo(x.y), s);
        s = fmaf(u[3], bf16hi(x.y), s);
        s = fmaf(u[4], bf16lo(x.z), s);
        s = fmaf(u[5], bf16hi(x.z), s);
        s = fmaf(u[6], bf16lo(x.w), s);
        return fmaf(u[7], bf16hi(x.w), s);
    }
};

template <int D, int NT, int G = 1, class KT = float, int ITER_OVERRIDE = 0>
struct GsCfg {
    static constexpr int NW = NT / 64;        // waves
    static constexpr int LPR = D * KRow<KT>::KB / 16;  // lanes per pooled-key row (16 bytes each)
    static constexpr int ROWS = NT / LPR;     // rows per workgroup-wide load
    // row loads in flight per thread (fewer where 1024 threads' registers also hold 8 query rows)
    static constexpr int ITER =
        ITER_OVERRIDE ? ITER_OVERRIDE : (NT >= 1024 && D == 128 && G >= 8 && KRow<KT>::KB == 4 ? 12 : 16);
    static constexpr int RPB = ROWS * ITER;   // rows per batch
    static constexpr int CH = D / 8;          // 16-byte bf16 chunks per weight row
    static constexpr int RG = NT / CH;        // weight-row groups
    static constexpr int WB = RG >= 128 ? 1 : 128 / RG;    // weight rows per thread per batch
    static constexpr int NBW = (256 + WB * RG - 1) / (WB * RG);  // batches covering dg <= 256
};

template <int D, int NT>
struct GsSmem {
    float a[256];                   // Wq qbar
    float u_part[GsCfg<D, NT>::NW][D];
    float u[D];
    SelBlockSmem<NT> sel;
};

struct GateSelectArgs {
    GateArgs gate;
    SelectPolicy pol;
    int k_max;
    int32_t *block_idx;  // [pairs, k_max]
    int32_t *n_sel;      // [pairs]
};

// sm.u = gate_scale * Wk^T (Wq qbar) of (b, g), qbar = mean of the group's
// query heads.  Loads are issued q, Wq, Wk, then whatever issue_rows() issues
// (the caller's pooled-key rows), so the dependent chain below (two small
// products, three barriers) runs while those rows are still arriving.  Weight
// rows past dg are clamped to the last one and masked, so no branch separates
// the loads.  Every thread of the NT-thread workgroup calls it.
template <int D, int G, int NT, class KT, class IssueRows>
__device__ __forceinline__ void gate_u(const GateArgs &ga, int b, int g, GsSmem<D, NT> &sm,
                                       IssueRows &&issue_rows) {
    using C = GsCfg<D, NT, G, KT>;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int dg = ga.dg;
    const int c = tid % C::CH, rg = tid / C::CH;
    const auto qrs = buffer_rsrc(ga.q + b * ga.sq_b + (int64_t)(g * G) * ga.sq_h,
                                 (uint32_t)(((int64_t)(G - 1) * ga.sq_h + D) * 2));
    const auto wqrs = buffer_rsrc(ga.wq + (int64_t)g * dg * D, (uint32_t)(dg * D * 2));
    const auto wkrs = buffer_rsrc(ga.wk + (int64_t)g * dg * D, (uint32_t)(dg * D * 2));
    uint4 qw[G];
#pragma unroll
    for (int h = 0; h < G; ++h) qw[h] = buf_ld16(qrs, (uint32_t)(h * ga.sq_h * 2) + c * 16, 0);
    auto wrow = [&](int r) { return (uint32_t)((r < dg ? r : dg - 1) * D * 2 + c * 16); };
    uint4 wqv[C::WB], wkv[C::WB];
#pragma unroll
    for (int i = 0; i < C::WB; ++i) wqv[i] = buf_ld16(wqrs, wrow(rg + i * C::RG), 0);
#pragma unroll
    for (int i = 0; i < C::WB; ++i) wkv[i] = buf_ld16(wkrs, wrow(rg + i * C::RG), 0);
    __builtin_amdgcn_sched_barrier(0);  // keep the issue order: the u inputs first
    issue_rows();
    __builtin_amdgcn_sched_barrier(0);

    float qb[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float f[8];
        unpack8(qw[h], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) qb[e] += f[e];
    }
    const float inv_g = 1.0f / (float)G;
#pragma unroll
    for (int e = 0; e < 8; ++e) qb[e] *= inv_g;
#pragma unroll
    for (int bw = 0; bw < C::NBW; ++bw) {  // a[r] = Wq[r] . qbar
        const int r0 = bw * C::WB * C::RG;
        if (bw > 0 && r0 >= dg) break;
        if (bw > 0) {
#pragma unroll
            for (int i = 0; i < C::WB; ++i) wqv[i] = buf_ld16(wqrs, wrow(r0 + rg + i * C::RG), 0);
        }
#pragma unroll
        for (int i = 0; i < C::WB; ++i) {
            const int r = r0 + rg + i * C::RG;
            float f[8];
            unpack8(wqv[i], f);
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) s = fmaf(f[e], qb[e], s);
            s = group_sum<C::CH>(s);  // the CH lanes of a row group share r
            if (c == 0 && r < dg) sm.a[r] = s;
        }
    }
    __syncthreads();
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int bw = 0; bw < C::NBW; ++bw) {  // u += a[r] * Wk[r]
        const int r0 = bw * C::WB * C::RG;
        if (bw > 0 && r0 >= dg) break;
        if (bw > 0) {
#pragma unroll
            for (int i = 0; i < C::WB; ++i) wkv[i] = buf_ld16(wkrs, wrow(r0 + rg + i * C::RG), 0);
        }
#pragma unroll
        for (int i = 0; i < C::WB; ++i) {
            const int r = r0 + rg + i * C::RG;
            float f[8];
            unpack8(wkv[i], f);
            const float ar = r < dg ? sm.a[r] : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = fmaf(ar, f[e], acc[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float s = cross_group_sum<C::CH>(acc[e]);  // row groups of this wave
        if (lane < C::CH) sm.u_part[wave][c * 8 + e] = s;
    }
    __syncthreads();
    if (tid < D) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < C::NW; ++w) s += sm.u_part[w][tid];
        sm.u[tid] = s * ga.gate_scale;
    }
    __syncthreads();
}

// Every thread of the NT-thread workgroup calls it; keys: LDS scratch of nb_max
// words.  G query heads per KV head; dg <= 256; KT the pooled keys' element type.
template <int D, int G, int NT, class Mem, class KT = float>
__device__ __forceinline__ void gate_select_pair(const GateSelectArgs &gs, int pair, GsSmem<D, NT> &sm,
                                                 uint32_t *keys) {
    using C = GsCfg<D, NT, G, KT>;
    using KR = KRow<KT>;
    const GateArgs &ga = gs.gate;
    const int tid = threadIdx.x;
    const int Hkv = ga.Hkv, nb_max = ga.nb_max;
    const int b = pair / Hkv, g = pair % Hkv;
    const int L = ga.seqlens[b];  // needed only once the scores exist

    // 1-2. u, with the first pooled-key rows in flight behind its inputs.  Row
    // indices past the table are clamped to its last row (their values are
    // discarded later), so none of these loads waits for the context length.
    const int lr = tid / C::LPR, lc = tid % C::LPR;
    const KT *kpool = reinterpret_cast<const KT *>(ga.kpool);
    const auto kprs = buffer_rsrc(kpool + (int64_t)pair * nb_max * D, (uint32_t)nb_max * D * KR::KB);
    auto krow = [&](int j) { return (uint32_t)((j < nb_max ? j : nb_max - 1) * D * KR::KB + lc * 16); };
    uint4 x[C::ITER];
    block_select_prepare<NT>(sm.sel);  // ordered before the selection by the barriers below
    gate_u<D, G, NT, KT>(ga, b, g, sm, [&] {
#pragma unroll
        for (int it = 0; it < C::ITER; ++it) x[it] = buf_ld16_nt(kprs, krow(lr + it * C::ROWS), 0);
    });

    // 3. score_j = u . kp_j for the complete blocks, batch by batch; -inf after them.
    int nc = (L < 0 ? 0 : L) / ga.block_size;
    nc = nc > nb_max ? nb_max : nc;
    nc = __builtin_amdgcn_readfirstlane(nc);
    float *srow = ga.scores + (int64_t)pair * nb_max;
    for (int j = nc + tid; j < nb_max; j += NT) Mem::stf(srow + j, -INFINITY);
    float uu[KR::EPL];
#pragma unroll
    for (int e = 0; e < KR::EPL; ++e) uu[e] = sm.u[lc * KR::EPL + e];
    for (int j0 = 0;;) {
#pragma unroll
        for (int it = 0; it < C::ITER; ++it) {
            const int j = j0 + lr + it * C::ROWS;
            float s = KR::dot(uu, x[it]);
            if constexpr (C::LPR == 8) {
                s = group_sum<8>(s);
            } else {
                s = group_sum<16>(s);
                if constexpr (C::LPR == 32) s = sum_xor16(s);
            }
            if (lc == 0 && j < nc) {
                Mem::stf(srow + j, s);
                keys[j] = order_key(s);
            }
        }
        j0 += C::RPB;
        if (j0 >= nc) break;
#pragma unroll
        for (int it = 0; it < C::ITER; ++it) x[it] = buf_ld16_nt(kprs, krow(j0 + lr + it * C::ROWS), 0);
    }
    __syncthreads();  // keys complete

    // 4. Selection: k blocks by the policy, ids ascending, -1 after.
    const int k = block_select_keys<NT, Mem>(keys, nc, gs.pol, gs.k_max, gs.block_idx + (int64_t)pair * gs.k_max,
                                             nullptr, sm.sel);
    if (tid == 0) Mem::sti(gs.n_sel + pair, k);
}

}  // namespace seer

