// decode_items.hpp -- device bodies of the sparse-decode split and its merge.
//
// Used by the standalone kernels (decode.hip), the per-head form (heads.hip)
// and the decode step (step.hip); the Mem policy (seer_device.hpp) says how
// data handed between launches is read and written.
//
// Operation ("SeerAttention-R: Sparse Attention Adaptation for Long
// Reasoning", abstract): a decoding kernel that reads only the KV blocks the
// gate kept.  For sequence b, KV head g and each query head h of g's group,
// softmax attention over T = (kept blocks) + (incomplete tail block).  The
// tail is always attended: it holds the current token and has no pooled key
// to be scored with.
//
// gfx950 design.  One workgroup (4 waves) per (split, KV head, sequence).  The
// pair's "units" (the kept blocks, then the tail) are cut into 32-token
// slices; a split owns a contiguous range of slices, dealt round-robin to its
// waves.  For each slice a wave does both products on v_mfma_f32_16x16x32_bf16
// with the group's query heads as the 16-wide N dimension (G <= 8 used):
//   loads : the wave's K and V rows of the slice go straight from HBM into its
//        LDS tiles (buffer_load ... lds, non-temporal, whole 256-byte rows per
//        16 lanes; the slice's first row is a scalar offset, rows past the
//        context re-read its last token).  A lane's 16 bytes land at base + 16 lane, so the
//        bank-conflict swizzles below are a choice of source chunk per lane.
//   QK : S^T = K Q^T, the K operand read from LDS (16-byte chunks XOR-swizzled
//        by row), the bf16 query a register operand.  Lane (g4, n) gets head
//        n's scores of tokens 16t + 4 g4 + 0..3, which is exactly its slice of
//        the P^T operand.
//   softmax : log2 domain, the scale folded into one FMA; one running max
//        per head, the same in the 4 lanes of the head, accumulators rescaled
//        only when some head's maximum moved.
//   PV : O^T = V^T P^T, the V^T operand read from the V tile (32-byte chunks
//        XOR-swizzled by row) with ds_read_b64_tr_b16.  P is split into bf16 high
//        and low parts (two MFMAs), so the products keep ~16 bits of the fp32
//        weights.
// At the end each wave's heads and then the 4 waves are combined, and the
// split writes (unnormalised o, running max, running sum) per head -- or,
// with a single split, the final normalised output directly.  A merge of the
// splits by log-sum-exp follows in a second kernel.
#pragma once

#include "seer_device.hpp"
#include "seer_host.hpp"
#include "topk_wave.hpp"

#include <math.h>

namespace seer {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));

// s_waitcnt immediate that waits until at most n vector-memory loads are
// outstanding (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt, lgkmcnt at max).
constexpr int vmcnt_wait(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

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
    static constexpr int TPW = 32;        // tokens of one slice: what a wave loads and attends at a time
    static constexpr int SPB = BS / TPW;  // slices per unit (4 for 128-token blocks, 2 for 64)
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

// LDS of one split: each wave's K and V rows of the current slice, and the
// per-wave partial results combined at the end (each wave's o [G][D] in its
// own K tile, which is free once its slices are done).
template <int D, int BS, int G>
struct DecodeSmem {
    using C = DecodeCfg<D, BS, G>;
    __attribute__((aligned(16))) uint16_t kt[C::NW][C::TPW * D];
    __attribute__((aligned(16))) uint16_t vt[C::NW][C::TPW * D];
    static_assert(G * D * sizeof(float) <= C::TPW * D * sizeof(uint16_t), "a wave's o fits its K tile");
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
// KL: the kept ids and their count come from LDS (kept, kept_n) instead of
// block_idx / n_sel.
template <int D, int BS, int G, class Mem, bool GT = false, bool PH = false, bool KL = false>
__device__ __forceinline__ void decode_split_item(const DecodeArgs &a, int split, int g, int b,
                                                  DecodeSmem<D, BS, G> &sm, uint32_t *dyn = nullptr,
                                                  const int32_t *kept = nullptr, int kept_n = 0) {
    using C = DecodeCfg<D, BS, G>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Wave w's per-head o, [G][D] floats in its own K tile (used there only after its slices).
    auto sm_o = [&](int w) { return reinterpret_cast<float (*)[D]>(sm.kt[w]); };
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
        // ids are clamped below both the complete blocks and the bitmap width nb_max
        const int id_hi = (nc < nb_max ? nc : nb_max) - 1;
        for (int i = tid; i < G * a.k_max; i += C::NT) {
            const int h = i / a.k_max, r = i % a.k_max;
            const int64_t row = (int64_t)b * a.Hq + g * G + h;
            int n = Mem::ldi(a.n_sel + row);
            n = n < 0 ? 0 : (n > kcap ? kcap : n);
            if (r < n && id_hi >= 0) {
                int id = Mem::ldi(a.block_idx + row * a.k_max + r);
                id = id < 0 ? 0 : (id > id_hi ? id_hi : id);
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
        nsel = GT ? kcap : (KL ? kept_n : Mem::ldi(a.n_sel + b * a.Hkv + g));
        nsel = nsel < 0 ? 0 : (nsel > kcap ? kcap : nsel);
    }
    // Each unit is SPB slices of 32 tokens; slice i is tokens 32 (i % SPB) ..
    // + 31 of unit i / SPB.  The S splits divide the pair's slices evenly, so
    // every split moves the same bytes to within one slice even when the units
    // do not divide by S; a unit at a split boundary is shared by two splits.
    // Within a split, wave w takes the slices i = w (mod NW): with 128-token
    // blocks always the unit's w-th quarter, with 64-token blocks half of
    // block 2 r + w / 2.  Either way a wave has 16 KiB of K and V in flight.
    constexpr int TPW = C::TPW, SPB = C::SPB;
    const int units = nsel + (tail > 0 ? 1 : 0);
    const int64_t nslices = (int64_t)units * SPB;
    const int i0 = (int)((split * nslices) / a.num_splits);  // this split's slices [i0, i1)
    const int i1 = (int)(((split + 1) * nslices) / a.num_splits);
    // This wave's rounds r: those whose slice r NW + wave lies in [i0, i1).
    const int r0 = __builtin_amdgcn_readfirstlane((i0 - wave + C::NW - 1) / C::NW);
    const int r1 = __builtin_amdgcn_readfirstlane((i1 - wave + C::NW - 1) / C::NW);

    constexpr int NKT = TPW / 16;  // 16-token tiles per slice
    constexpr int KS = D / 32;     // k-steps of S^T = K Q^T
    constexpr int DT = D / 16;     // 16-wide d tiles of O^T
    constexpr int CPR = D / 8;     // 16-byte chunks per row
    constexpr int RPD = 64 / CPR;  // rows per 1 KiB LDS load
    constexpr int NDMA = TPW / RPD;
    constexpr int XM = CPR / 2 - 1;  // 32-byte chunk swizzle mask
    static_assert(G <= 16 && TPW == 32 && SPB * TPW == BS, "MFMA decode tile");
    const int g4 = lane >> 4, n = lane & 15;

    // Q operand: lane (g4, n) holds dims 8 g4 + 32 ks .. + 7 of head n (zero for n >= G).
    bf16x8_t qop[KS];
    const uint16_t *qb = a.q + b * a.sq_b + (int64_t)(g * G) * a.sq_h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qop[ks] = __builtin_bit_cast(bf16x8_t, n < G ? ldg16(qb + n * a.sq_h + 8 * g4 + 32 * ks) : make_uint4(0, 0, 0, 0));

    // K/V of (b, g) through buffer descriptors: a slice's first row is a scalar
    // byte offset, each lane's rows and chunks a fixed 32-bit offset.
    const uint16_t *kb = a.k + b * a.skv_b + g * a.skv_h;
    const uint16_t *vb = a.v + b * a.skv_b + g * a.skv_h;
    const uint32_t region = (uint32_t)((int64_t)a.kv_capacity * a.skv_t * 2);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)kb, 0, region, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)vb, 0, region, kBufferFlags);
    const int32_t *sel = (GT || PH || KL) ? nullptr : a.block_idx + (int64_t)(b * a.Hkv + g) * a.k_max;
    // Tiles: lane l of load q fills LDS row rr = q RPD + l / CPR, 16-byte slot
    // s = l % CPR.  K slot s holds chunk s ^ (rr & (CPR - 1)); V slot s holds
    // the chunk whose 32-byte pair lands there when pairs are XORed with rr & XM.
    uint32_t kof[NDMA], vof[NDMA];
#pragma unroll
    for (int q = 0; q < NDMA; ++q) {
        const int rr = q * RPD + lane / CPR, s = lane % CPR;
        const int kc = s ^ (rr & (CPR - 1));
        const int vc = ((((s >> 1) ^ (rr & XM)) << 1) | (s & 1));
        kof[q] = (uint32_t)((rr * a.skv_t + kc * 8) * 2);
        vof[q] = (uint32_t)((rr * a.skv_t + vc * 8) * 2);
    }
    char *const kt = reinterpret_cast<char *>(sm.kt[wave]);
    char *const vt = reinterpret_cast<char *>(sm.vt[wave]);
    // K operand reads: lane (g4, n) takes row 16t + n, chunk g4 + 4 ks.
    const char *const kr0 = kt + n * (D * 2);
    // Transposing reads: lane (g4, s) points at tile row 16t + 4 g4 + s / 4,
    // columns 16 dt + 4 (s % 4) + 0..3; the row's swizzle does not depend on t.
    const int trow = 4 * g4 + (n >> 2), tx = trow & XM;
    const char *const vr0 = vt + trow * (D * 2) + (n & 3) * 8;

    f32x4_t oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_part = 0.f;  // of head n

    int ids = 0, id0 = -(1 << 30);  // kept block ids of units [id0, id0 + 64), one per lane
    for (int r = r0; r < r1; ++r) {
        const int sl = r * C::NW + wave;  // this wave's slice of the round
        const int u = sl / SPB;           // its unit
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
                    if constexpr (KL)
                        ids = u + lane < nsel ? kept[u + lane] : 0;
                    else
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
        const int wt0 = (sl % SPB) * TPW;  // first token of this slice inside its unit
        if constexpr (!GT) {
            if (wt0 >= cnt) continue;  // a slice of the tail past the context: nothing to attend
        }
        const uint32_t soff = (uint32_t)(tok0 + wt0) * (uint32_t)a.skv_t * 2u;
        // The tail unit's rows at or past the context end re-read its last token:
        // they take no weight, and they are neither read past the cache (the range
        // check covers only the per-lane offset) nor able to bring a non-finite
        // value of unused cache rows into the P V product (0 * inf is NaN).
        uint32_t ko[NDMA], vo[NDMA];
#pragma unroll
        for (int q = 0; q < NDMA; ++q) {
            ko[q] = kof[q];
            vo[q] = vof[q];
        }
        if (cnt < BS) {
#pragma unroll
            for (int q = 0; q < NDMA; ++q) {
                const int over = wt0 + q * RPD + lane / CPR - (cnt - 1);
                const uint32_t back = over > 0 ? (uint32_t)over * (uint32_t)a.skv_t * 2u : 0u;
                ko[q] -= back;
                vo[q] -= back;
            }
        }
        // This wave's K and V rows into its LDS tiles (the previous unit's reads of
        // them are complete: their results fed the previous unit's MFMAs).
#pragma unroll
        for (int q = 0; q < NDMA; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void *)(kt + q * 1024), 16,
                                                     (int)ko[q], (int)soff, 0, 2);
#pragma unroll
        for (int q = 0; q < NDMA; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void *)(vt + q * 1024), 16,
                                                     (int)vo[q], (int)soff, 0, 2);
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(NDMA));  // the K rows are in LDS

        // S^T tiles: lane (g4, n) gets head n's raw scores of tokens 16t + 4 g4 + i.
        f32x4_t s[NKT];
#pragma unroll
        for (int t = 0; t < NKT; ++t) {
            s[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8_t kop = *reinterpret_cast<const bf16x8_t *>(
                    kr0 + t * 16 * (D * 2) + (((g4 + 4 * ks) ^ (n & (CPR - 1))) << 4));
                s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[ks], s[t], 0, 0, 0);
            }
        }
        if (cnt < BS) {  // the tail unit: rows past the context take no weight
#pragma unroll
            for (int t = 0; t < NKT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) s[t][i] = wt0 + 16 * t + 4 * g4 + i < cnt ? s[t][i] : -INFINITY;
        }
        if constexpr (PH) {  // heads that did not keep this block give it no weight
            if (!((hmask >> n) & 1u)) {
#pragma unroll
                for (int t = 0; t < NKT; ++t) s[t] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            }
        }

        // Running max per head (log2 domain), rescale factor, weights.
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmax_fast(mx, s[t][i]);
        mx = max_xor32(max_xor16(mx)) * a.scale_log2;  // the head's 4 lanes; the host checks the scale is > 0
        const float m_new = fmax_fast(m_run, mx);
        const float m_ref = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_ref);
        m_run = m_new;
        float lsum = 0.f;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s[t][i] = fast_exp2(fmaf(s[t][i], a.scale_log2, -m_ref));
                lsum += s[t][i];
            }
        l_part = l_part * alpha + lsum;
        if constexpr (GT) {  // log2-sum-exp of the slice, entry sl % SPB of the unit's 4
            const float lw = sum_xor32(sum_xor16(lsum));
            if (g4 == 0 && n < G)
                a.blk_lse[(((int64_t)(b * a.Hkv + g) * a.units_max + u) * G + n) * 4 + sl % SPB] =
                    lw > 0.f ? m_ref + log2f(lw) : -INFINITY;
        }
        if (__ballot(alpha != 1.0f)) {  // some head's maximum moved
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
        }

        // P^T operands, high and low bf16 parts: k-slots 8 g4 + 4t + i <- token 16t + 4 g4 + i.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's V rows are in LDS
        bf16x8_t ph, pl;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const __bf16 hi = (__bf16)s[t][i];
                ph[4 * t + i] = hi;
                pl[4 * t + i] = (__bf16)(s[t][i] - (float)hi);
            }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const char *p = vr0 + ((dt ^ tx) << 5);
            const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)p);
            const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s *)(p + 16 * D * 2));
            const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, ph, oacc[dt], 0, 0, 0);
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pl, oacc[dt], 0, 0, 0);
        }
        // The next unit's loads overwrite the tile: keep them behind this unit's reads.
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
    }

    // This wave's per-head results: the sum over the head's 4 lanes; O^T tile dt
    // holds rows d = 16 dt + 4 g4 + i of head n.
    const float l_tot = sum_xor32(sum_xor16(l_part));
    if (n < G) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sm_o(wave)[n][16 * dt + 4 * g4 + i] = oacc[dt][i];
        if (g4 == 0) {
            sm_m[wave][n] = m_run;
            sm_l[wave][n] = l_tot;
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
            O = fmaf(sm_o(w)[h][e], f, O);
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
    // The first PRE partial rows do not depend on (m, l): they are requested
    // together with them, one memory round trip instead of two.
    constexpr int PRE = 8;
    const float *po = part_o + bh * S * D + (tid < D ? tid : 0);
    float x0[PRE];
    if (tid < D) {
#pragma unroll
        for (int i = 0; i < PRE; ++i) x0[i] = i < S ? Mem::ldf(po + (int64_t)i * D) : 0.f;
    }
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
        float O = 0.f;
#pragma unroll
        for (int i = 0; i < PRE; ++i)
            if (i < S) O = fmaf(x0[i], sm.w[i], O);
        int sp = PRE;
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
