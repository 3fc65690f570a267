// decode_items.hpp -- device bodies of the sparse-decode split and its merge.
//
// Used by the standalone kernels (decode.hip) and by the fused one-launch
// decode step (step.hip); the Mem policy (seer_device.hpp) says how data
// handed to another workgroup is written and read.
//
// Operation ("SeerAttention-R: Sparse Attention Adaptation for Long
// Reasoning", abstract): a decoding kernel that reads only the KV blocks the
// gate kept.  For sequence b, KV head g and each query head h of g's group,
// softmax attention over T = (kept blocks) + (incomplete tail block).  The
// tail is always attended: it holds the current token and has no pooled key
// to be scored with.
//
// gfx950 design.  One workgroup (4 waves) per (split, KV head, sequence).  A
// split owns a contiguous range of "units" (a kept block, or the tail).  For
// every unit each wave takes a quarter of the block's tokens:
//   loads : non-temporal 16-byte buffer loads; the unit's first row is a
//        scalar offset, each lane's rows a fixed 32-bit offset, and rows past
//        the cache read as zero (the descriptor's range check).
//   QK : 8 lanes per key row, each lane a 16-byte chunk per 64 head dims;
//        v_dot2_f32_bf16 with the bf16 query held in registers, then an
//        8-lane DPP all-reduce.  The key bytes feed all G query heads.
//   softmax : log2 domain, the scale folded into one FMA; one running max
//        per head that is uniform across the wave, so partial sums need no
//        rescaling when the wave's lane groups are combined, and the
//        accumulators are rescaled only when some head's maximum moved.
//   PV : probabilities go through LDS to a second layout, one 16-byte value
//        chunk per lane (a whole 256-byte row per 16 lanes, fully coalesced),
//        fp32 FMA into G x 8 accumulators per lane.
// At the end the wave's lane groups and then the 4 waves are combined, and
// the split writes (unnormalised o, running max, running sum) per head -- or,
// with a single split, the final normalised output directly.  A merge of the
// splits by log-sum-exp follows (a second kernel, or later work items of the
// fused step).
#pragma once

#include "seer_device.hpp"
#include "seer_host.hpp"
#include "topk_wave.hpp"

#include <math.h>

namespace seer {

struct DecodeArgs {
    const uint16_t *q;
    int64_t sq_b, sq_h;
    const uint16_t *k, *v;
    int64_t skv_b, skv_h, skv_t;
    int kv_capacity;
    const int32_t *seqlens, *block_idx, *n_sel;
    int k_max, Hq, Hkv, num_splits;
    float scale_log2;          // softmax_scale * log2(e)
    float *part_o;             // [B][Hq][S][D]
    float2 *part_ml;           // [B][Hq][S] (running max in log2 units, running sum)
    void *out;
    int out_dtype;
    float *lse;
    // Ground-truth form only: per (b, KV head, unit, head, wave) log2 of the
    // wave's sum of exp over the unit's tokens, at a stride of units_max units.
    // Per-head form: units_max is the pooled-table width nb_max.
    float *blk_lse;
    int units_max;
};

// Per-head form: LDS words the union of a group's block sets needs (bitmaps,
// ascending union ids, per-id head masks).
__host__ __device__ inline int heads_union_cap(int nb_max, int G, int k_max) {
    const int64_t c = (int64_t)G * k_max;
    return (int)(c < nb_max ? c : nb_max);
}
__host__ __device__ inline int heads_union_words(int nb_max, int G, int k_max) {
    return G * ((nb_max + 31) / 32) + 2 * heads_union_cap(nb_max, G, k_max);
}

template <int D, int BS, int G>
struct DecodeCfg {
    static constexpr int NT = 256, NW = 4;
    static constexpr int CH = D / 8;          // 16-byte chunks per row
    static constexpr int LPR = 8;             // QK: lanes per key row
    static constexpr int ROWS = 64 / LPR;     // key rows per wave-wide load
    static constexpr int CPL = CH / LPR;      // key chunks per lane
    static constexpr int TPW = BS / NW;       // tokens per wave per unit
    static constexpr int TPL = TPW / ROWS;    // key rows per lane per unit
    static constexpr int LPV = CH;            // PV: lanes per value row (one chunk each)
    static constexpr int ROWSV = 64 / LPV;    // value rows per wave-wide load
    static constexpr int TPLV = TPW / ROWSV;  // value rows per lane per unit
    static_assert(CPL >= 1 && TPL >= 1 && TPLV >= 1, "tile shape");
};

__device__ __forceinline__ uint4 ldg16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ uint4 ldg16_stream(const uint16_t *p) {
    const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ void store_out(void *out, int dtype, int64_t i, float x) {
    if (dtype == SEER_OUT_F32)
        static_cast<float *>(out)[i] = x;
    else
        static_cast<uint16_t *>(out)[i] = f32_to_bf16(x);
}

// LDS of one split: probabilities handed from the QK to the PV layout, and the
// per-wave partial results combined at the end.
template <int D, int BS, int G>
struct DecodeSmem {
    using C = DecodeCfg<D, BS, G>;
    float p[C::NW][C::TPW][G];
    float o[C::NW][G][D];
    float m[C::NW][G], l[C::NW][G];
    int n_union;  // per-head form: size of the group's union of kept blocks
};

// One split of one (b, KV head g): attention of the group's query heads over
// its units.  Writes the split's (o, m, l) through Mem, or with a single split
// the normalised output.  Every thread of the 256-thread workgroup calls it.
// GT (the ground-truth form): every complete block is a unit (up to k_max of
// them, in order) and each unit's per-wave log-sum-exp goes to a.blk_lse.
// PH (the per-head form): block_idx / n_sel hold one set per query head; the
// units are the union of the group's sets, ascending, and a head gives no
// weight to a unit it did not keep (dyn: heads_union_words(...) LDS words).
template <int D, int BS, int G, class Mem, bool GT = false, bool PH = false>
__device__ __forceinline__ void decode_split_item(const DecodeArgs &a, int split, int g, int b,
                                                  DecodeSmem<D, BS, G> &sm, uint32_t *dyn = nullptr) {
    using C = DecodeCfg<D, BS, G>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane / C::LPR, c = lane % C::LPR;      // QK layout
    const int rv = lane / C::LPV, cv = lane % C::LPV;    // PV layout
    auto &p_lds = sm.p;
    auto &sm_o = sm.o;
    auto &sm_m = sm.m;
    auto &sm_l = sm.l;

    int L = a.seqlens[b];
    L = L < 0 ? 0 : (L > a.kv_capacity ? a.kv_capacity : L);
    const int nc = L / BS, tail = L - nc * BS;
    const int kcap = a.k_max < nc ? a.k_max : nc;
    int nsel = 0;
    uint32_t *uid = nullptr, *umask = nullptr;
    if constexpr (PH) {
        // Union of the G heads' sets: one bitmap per head, then wave 0 lists the
        // set bits in ascending order with the mask of the heads that kept each.
        const int nb_max = a.units_max, W = (nb_max + 31) / 32;
        uint32_t *bm = dyn;
        uid = dyn + G * W;
        umask = uid + heads_union_cap(nb_max, G, a.k_max);
        for (int i = tid; i < G * W; i += C::NT) bm[i] = 0u;
        __syncthreads();
        for (int i = tid; i < G * a.k_max; i += C::NT) {
            const int h = i / a.k_max, r = i % a.k_max;
            const int64_t row = (int64_t)b * a.Hq + g * G + h;
            int n = Mem::ldi(a.n_sel + row);
            n = n < 0 ? 0 : (n > kcap ? kcap : n);
            if (r < n) {
                int id = Mem::ldi(a.block_idx + row * a.k_max + r);
                id = id < 0 ? 0 : (id >= nc ? nc - 1 : id);
                atomicOr(&bm[h * W + id / 32], 1u << (id % 32));
            }
        }
        __syncthreads();
        if (wave == 0) {
            int base = 0;
            for (int w0 = 0; w0 < W; w0 += 64) {
                const int w = w0 + lane;
                uint32_t bits[G], uni = 0u;
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    bits[h] = w < W ? bm[h * W + w] : 0u;
                    uni |= bits[h];
                }
                const int cnt = __popc(uni);
                const int incl = wave_inclusive_scan(cnt, lane);
                int pos = base + incl - cnt;
                while (uni) {
                    const int bit = __builtin_ctz(uni);
                    uni &= uni - 1u;
                    uint32_t m = 0u;
#pragma unroll
                    for (int h = 0; h < G; ++h) m |= ((bits[h] >> bit) & 1u) << h;
                    uid[pos] = (uint32_t)(w * 32 + bit);
                    umask[pos] = m;
                    ++pos;
                }
                base += __builtin_amdgcn_readlane(incl, 63);
            }
            if (lane == 0) sm.n_union = base;
        }
        __syncthreads();
        nsel = __builtin_amdgcn_readfirstlane(sm.n_union);
    } else {
        nsel = GT ? kcap : Mem::ldi(a.n_sel + b * a.Hkv + g);
        nsel = nsel < 0 ? 0 : (nsel > kcap ? kcap : nsel);
    }
    const int units = nsel + (tail > 0 ? 1 : 0);
    const int u0 = (int)(((int64_t)split * units) / a.num_splits);
    const int u1 = (int)(((int64_t)(split + 1) * units) / a.num_splits);

    // Query rows of the group, bf16 pairs, the chunks this lane multiplies.
    uint4 qv[G][C::CPL];
    const uint16_t *qb = a.q + b * a.sq_b + (int64_t)(g * G) * a.sq_h;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < C::CPL; ++i) qv[h][i] = ldg16(qb + h * a.sq_h + (c + i * C::LPR) * 8);

    float m_run[G], l_part[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_run[h] = -INFINITY;
        l_part[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
    }

    // K/V of (b, g) through buffer descriptors: a unit's first row is a scalar
    // byte offset, each lane's rows and chunks a fixed 32-bit offset.
    const uint16_t *kb = a.k + b * a.skv_b + g * a.skv_h;
    const uint16_t *vb = a.v + b * a.skv_b + g * a.skv_h;
    const uint32_t region = (uint32_t)((int64_t)a.kv_capacity * a.skv_t * 2);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)kb, 0, region, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)vb, 0, region, kBufferFlags);
    const int32_t *sel = (GT || PH) ? nullptr : a.block_idx + (int64_t)(b * a.Hkv + g) * a.k_max;
    const int wt0 = wave * C::TPW;  // first token of this wave inside a unit
    uint32_t koff[C::TPL][C::CPL], voff[C::TPLV];
#pragma unroll
    for (int t = 0; t < C::TPL; ++t)
#pragma unroll
        for (int i = 0; i < C::CPL; ++i)
            koff[t][i] = (uint32_t)(((wt0 + r + t * C::ROWS) * a.skv_t + (c + i * C::LPR) * 8) * 2);
#pragma unroll
    for (int t = 0; t < C::TPLV; ++t) voff[t] = (uint32_t)(((wt0 + rv + t * C::ROWSV) * a.skv_t + cv * 8) * 2);

    int ids = 0, id0 = u0 - 64;  // kept block ids of units [id0, id0 + 64), one per lane
    for (int u = u0; u < u1; ++u) {
        int tok0, cnt;
        uint32_t hmask = (1u << G) - 1u;  // heads that take this unit
        if (u < nsel) {
            int blk = u;
            if constexpr (PH) {
                blk = (int)uid[u];
                hmask = __builtin_amdgcn_readfirstlane(umask[u]);
            } else if constexpr (!GT) {
                if (u - id0 >= 64) {
                    id0 = u;
                    ids = u + lane < nsel ? Mem::ldi(sel + u + lane) : 0;
                }
                blk = __builtin_amdgcn_readlane(ids, u - id0);
                blk = blk < 0 ? 0 : (blk >= nc ? nc - 1 : blk);
            }
            tok0 = blk * BS;
            cnt = BS;
        } else {
            tok0 = nc * BS;
            cnt = tail;
        }
        tok0 = __builtin_amdgcn_readfirstlane(tok0);
        cnt = __builtin_amdgcn_readfirstlane(cnt);
        // Rows past the end of the cache read as zero (buffer range check) and,
        // like rows past cnt, are masked out of the softmax.
        const uint32_t soff = (uint32_t)tok0 * (uint32_t)a.skv_t * 2u;
        uint4 kr[C::TPL][C::CPL], vr[C::TPLV];
#pragma unroll
        for (int t = 0; t < C::TPL; ++t)
#pragma unroll
            for (int i = 0; i < C::CPL; ++i) kr[t][i] = buf_ld16_nt(krs, koff[t][i], soff);
#pragma unroll
        for (int t = 0; t < C::TPLV; ++t) vr[t] = buf_ld16_nt(vrs, voff[t], soff);

        // Raw scores q.k of this lane group's key rows for every head.
        float s[C::TPL][G];
#pragma unroll
        for (int t = 0; t < C::TPL; ++t)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < C::CPL; ++i) {
                    acc = dot2_bf16(qv[h][i].x, kr[t][i].x, acc);
                    acc = dot2_bf16(qv[h][i].y, kr[t][i].y, acc);
                    acc = dot2_bf16(qv[h][i].z, kr[t][i].z, acc);
                    acc = dot2_bf16(qv[h][i].w, kr[t][i].w, acc);
                }
                s[t][h] = group_sum<C::LPR>(acc);
            }
        if (cnt < BS) {  // the tail unit: rows past the context take no weight
#pragma unroll
            for (int t = 0; t < C::TPL; ++t)
#pragma unroll
                for (int h = 0; h < G; ++h) s[t][h] = wt0 + r + t * C::ROWS < cnt ? s[t][h] : -INFINITY;
        }
        if constexpr (PH) {  // heads that did not keep this block give it no weight
#pragma unroll
            for (int h = 0; h < G; ++h)
                if (!((hmask >> h) & 1u)) {
#pragma unroll
                    for (int t = 0; t < C::TPL; ++t) s[t][h] = -INFINITY;
                }
        }

        // Wave-uniform running max per head (log2 domain), rescale factors, probabilities.
        float alpha[G];
        bool rescale = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mx = s[0][h];
#pragma unroll
            for (int t = 1; t < C::TPL; ++t) mx = fmax_fast(mx, s[t][h]);
            mx = cross_group_max<C::LPR>(mx) * a.scale_log2;  // the scale is positive
            const float m_new = fmax_fast(m_run[h], mx);
            const float m_ref = m_new == -INFINITY ? 0.f : m_new;
            alpha[h] = fast_exp2(m_run[h] - m_ref);
            rescale |= alpha[h] != 1.0f;
            m_run[h] = m_new;
            float lsum = 0.f;
#pragma unroll
            for (int t = 0; t < C::TPL; ++t) {
                s[t][h] = fast_exp2(fmaf(s[t][h], a.scale_log2, -m_ref));
                lsum += s[t][h];
            }
            l_part[h] = l_part[h] * alpha[h] + lsum;
            if constexpr (GT) {  // this wave's log2-sum-exp of the unit (its quarter of the tokens)
                const float lw = cross_group_sum<C::LPR>(lsum);
                if (lane == 0)
                    a.blk_lse[(((int64_t)(b * a.Hkv + g) * a.units_max + u) * G + h) * C::NW + wave] =
                        lw > 0.f ? m_ref + log2f(lw) : -INFINITY;
            }
        }

        // Probabilities to LDS (one writer per key row), then back in the PV layout.
        if (c == 0) {
#pragma unroll
            for (int t = 0; t < C::TPL; ++t)
#pragma unroll
                for (int h = 0; h < G; ++h) p_lds[wave][r + t * C::ROWS][h] = s[t][h];
        }
        // LDS accesses of one wave complete in issue order; only this wave reads its slice.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        if (rescale) {  // wave-uniform: the running maxima are the same in every lane
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) o[h][e] *= alpha[h];
        }
        // PV in fp32: one 16-byte value chunk per lane, every head's probability from LDS.
#pragma unroll
        for (int t = 0; t < C::TPLV; ++t) {
            float p[G];
#pragma unroll
            for (int h = 0; h < G; ++h) p[h] = p_lds[wave][rv + t * C::ROWSV][h];
            const uint32_t w4[4] = {vr[t].x, vr[t].y, vr[t].z, vr[t].w};
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const float v0 = bf16lo(w4[e2]), v1 = bf16hi(w4[e2]);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    o[h][2 * e2] = fmaf(p[h], v0, o[h][2 * e2]);
                    o[h][2 * e2 + 1] = fmaf(p[h], v1, o[h][2 * e2 + 1]);
                }
            }
        }
        // The next unit overwrites p_lds; keep this unit's reads ahead of it.
        __builtin_amdgcn_wave_barrier();
    }

    // Combine the wave's lane groups: sums only, the max is already wave-uniform.
#pragma unroll
    for (int h = 0; h < G; ++h) {
        l_part[h] = cross_group_sum<C::LPR>(l_part[h]);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = cross_group_sum<C::LPV>(o[h][e]);
    }
    if (rv == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) sm_o[wave][h][cv * 8 + e] = o[h][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            sm_m[wave][h] = m_run[h];
            sm_l[wave][h] = l_part[h];
        }
    }
    __syncthreads();

    // Combine the 4 waves and emit this split's result.
    for (int i = tid; i < G * D; i += C::NT) {
        const int h = i / D, e = i % D;
        float M = sm_m[0][h];
#pragma unroll
        for (int w = 1; w < C::NW; ++w) M = fmax_fast(M, sm_m[w][h]);
        const float Mref = M == -INFINITY ? 0.f : M;
        float O = 0.f, Ls = 0.f;
#pragma unroll
        for (int w = 0; w < C::NW; ++w) {
            const float f = fast_exp2(sm_m[w][h] - Mref);
            O = fmaf(sm_o[w][h][e], f, O);
            Ls = fmaf(sm_l[w][h], f, Ls);
        }
        const int hq = g * G + h;
        const int64_t bh = (int64_t)b * a.Hq + hq;
        if (a.num_splits == 1) {
            store_out(a.out, a.out_dtype, bh * D + e, Ls > 0.f ? O / Ls : 0.f);
            if (e == 0 && a.lse) a.lse[bh] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
        } else {
            Mem::stf(a.part_o + (bh * a.num_splits + split) * D + e, O);
            if (e == 0) Mem::stf2(a.part_ml + bh * a.num_splits + split, M, Ls);
        }
    }
}

// Log-sum-exp merge of the splits of one (b, query head) = row bh, by the first
// 128 threads of the workgroup (the others only take part in the barriers):
// split maxima and sums loaded in parallel, the weights 2^(m_s - M) staged in
// LDS, then each output column summed over the splits with independent loads.
constexpr int kMaxSplits = 128;

struct MergeSmem {
    float w[kMaxSplits];
    float red[2][2];
};

template <int D, class Mem>
__device__ __forceinline__ void decode_merge_row(const float *part_o, const float2 *part_ml, int S, int64_t bh,
                                                 void *out, int out_dtype, float *lse, MergeSmem &sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float2 v = make_float2(-INFINITY, 0.f);
    if (tid < S) v = Mem::ldf2(part_ml + bh * S + tid);
    float M = wave_max(v.x);
    if (lane == 0 && wave < 2) sm.red[0][wave] = M;
    __syncthreads();
    M = fmax_fast(sm.red[0][0], sm.red[0][1]);
    const float Mref = M == -INFINITY ? 0.f : M;
    const float f = tid < S ? fast_exp2(v.x - Mref) : 0.f;
    if (tid < S) sm.w[tid] = f;
    float Ls = wave_sum(v.y * f);
    if (lane == 0 && wave < 2) sm.red[1][wave] = Ls;
    __syncthreads();
    Ls = sm.red[1][0] + sm.red[1][1];
    if (tid < D) {
        const float *po = part_o + bh * S * D + tid;
        float O = 0.f;
        int sp = 0;
        for (; sp + 8 <= S; sp += 8) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = Mem::ldf(po + (int64_t)(sp + i) * D);
#pragma unroll
            for (int i = 0; i < 8; ++i) O = fmaf(x[i], sm.w[sp + i], O);
        }
        for (; sp < S; ++sp) O = fmaf(Mem::ldf(po + (int64_t)sp * D), sm.w[sp], O);
        store_out(out, out_dtype, bh * D + tid, Ls > 0.f ? O / Ls : 0.f);
        if (tid == 0 && lse) lse[bh] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
    }
    __syncthreads();  // the weights in LDS may be reused by the caller's next row
}

}  // namespace seer
