// gate_heads_items.hpp -- per-query-head gate scores and selection of one
// (b, KV head) by one workgroup: the alternative to the shared group selection.
//
// Every query head h of the group keeps its own top-k blocks by its own gate
// score s_hj = gate_scale * (Wq q_h) . (Wk kp_j) (the SeerAttention gate of
// "SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs", abstract
// v1, without the group mean).  As in gate_select_items.hpp the q and weight
// loads are issued before the pooled-key rows; u_h = gate_scale * Wk^T (Wq q_h)
// is formed head by head from the weight rows held in registers; each pooled
// row, loaded once, is multiplied with all G vectors; the scores of head h go
// to the output row (b, g*G + h) and, as order-preserving keys, to LDS; wave h
// then selects head h's blocks (the one-wave radix select of topk_wave.hpp).
#pragma once

#include "gate_select_items.hpp"

namespace seer {

template <int D, int NT, int G>
struct GhSmem {
    float a[G][256];                    // Wq q_h
    float u_part[GsCfg<D, NT>::NW][D];
    float u[G][D];
    int hist[G][256];                   // one selection histogram per head's wave
};

// scores [B][Hq][nb_max], block_idx [B][Hq][k_max], n_sel [B][Hq].  keys: LDS
// scratch of G * nb_max words.  Every thread of the NT-thread workgroup calls it.
template <int D, int G, int NT, class Mem>
__device__ __forceinline__ void gate_select_heads_pair(const GateSelectArgs &gs, int pair, GhSmem<D, NT, G> &sm,
                                                       uint32_t *keys) {
    static_assert(G <= NT / 64, "one wave per head for the selection");
    using C = GsCfg<D, NT, G, float, G >= 4 ? 8 : 16>;  // fewer rows in flight: G score vectors in registers
    const GateArgs &ga = gs.gate;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Hkv = ga.Hkv, dg = ga.dg, nb_max = ga.nb_max;
    const int b = pair / Hkv, g = pair % Hkv;
    const int L = ga.seqlens[b];

    // 1. Loads: the group's query rows, first weight rows, first pooled-key rows.
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
    const int lr = tid / C::LPR, lc = tid % C::LPR;
    const auto kprs = buffer_rsrc(ga.kpool + (int64_t)pair * nb_max * D, (uint32_t)nb_max * D * 4);
    auto krow = [&](int j) { return (uint32_t)((j < nb_max ? j : nb_max - 1) * D * 4 + lc * 16); };
    uint4 x[C::ITER];
#pragma unroll
    for (int it = 0; it < C::ITER; ++it) x[it] = buf_ld16_nt(kprs, krow(lr + it * C::ROWS), 0);
    __builtin_amdgcn_sched_barrier(0);

    // 2. a_h = Wq q_h for every head, then u_h = gate_scale * Wk^T a_h head by head.
#pragma unroll
    for (int bw = 0; bw < C::NBW; ++bw) {
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
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float qf[8];
                unpack8(qw[h], qf);
                float s = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) s = fmaf(f[e], qf[e], s);
                s = group_sum<C::CH>(s);  // the CH lanes of a row group share r
                if (c == 0 && r < dg) sm.a[h][r] = s;
            }
        }
    }
    __syncthreads();
    for (int h = 0; h < G; ++h) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int bw = 0; bw < C::NBW; ++bw) {
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
                const float ar = r < dg ? sm.a[h][r] : 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = fmaf(ar, f[e], acc[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float s = cross_group_sum<C::CH>(acc[e]);
            if (lane < C::CH) sm.u_part[wave][c * 8 + e] = s;
        }
        __syncthreads();
        if (tid < D) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < C::NW; ++w) s += sm.u_part[w][tid];
            sm.u[h][tid] = s * ga.gate_scale;
        }
        __syncthreads();
    }

    // 3. s_hj = u_h . kp_j for the complete blocks; -inf after them.
    int nc = (L < 0 ? 0 : L) / ga.block_size;
    nc = nc > nb_max ? nb_max : nc;
    nc = __builtin_amdgcn_readfirstlane(nc);
    float *srow = ga.scores + ((int64_t)b * Hkv * G + (int64_t)g * G) * nb_max;  // row of head g*G + 0
    for (int i = tid; i < G * (nb_max - nc); i += NT) {
        const int h = i / (nb_max - nc), j = nc + i % (nb_max - nc);
        Mem::stf(srow + (int64_t)h * nb_max + j, -INFINITY);
    }
    float uu[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) uu[h][e] = sm.u[h][lc * 4 + e];
    for (int j0 = 0;;) {
#pragma unroll
        for (int it = 0; it < C::ITER; ++it) {
            const int j = j0 + lr + it * C::ROWS;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float s = KRow<float>::dot(uu[h], x[it]);
                s = group_sum<16>(s);
                if constexpr (C::LPR == 32) s = sum_xor16(s);
                if (lc == 0 && j < nc) {
                    Mem::stf(srow + (int64_t)h * nb_max + j, s);
                    keys[h * nb_max + j] = order_key(s);
                }
            }
        }
        j0 += C::RPB;
        if (j0 >= nc) break;
#pragma unroll
        for (int it = 0; it < C::ITER; ++it) x[it] = buf_ld16_nt(kprs, krow(j0 + lr + it * C::ROWS), 0);
    }
    __syncthreads();  // keys complete

    // 4. Wave h selects head h's k = min(k_max, nc) blocks.
    if (wave < G) {
        const int h = wave, k_max = gs.k_max;
        const int k = k_max < nc ? k_max : nc;
        const int64_t row = (int64_t)b * Hkv * G + (int64_t)g * G + h;
        int32_t *out = gs.block_idx + row * k_max;
        if (k == nc || k == 0) {
            for (int i = lane; i < k_max; i += 64) Mem::sti(out + i, i < k ? i : -1);
        } else {
            wave_topk_from_keys<Mem>(nc, k, keys + h * nb_max, sm.hist[h], out, lane);
            for (int i = k + lane; i < k_max; i += 64) Mem::sti(out + i, -1);
        }
        if (lane == 0) Mem::sti(gs.n_sel + row, k);
    }
}

}  // namespace seer
