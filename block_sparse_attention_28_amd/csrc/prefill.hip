// prefill.hip -- SeerAttention block-sparse causal prefill: gate and attention.
//
// Operation ("SeerAttention: Learning Intrinsic Sparse Attention in Your
// LLMs", abstract v1): the gate pools Q and K along the sequence, one vector
// per bs-token block, projects both through learnable linear layers and
// multiplies the results into block scores; a block-sparse FlashAttention
// kernel then attends only the activated blocks.  Here row i of the causal
// block mask keeps its diagonal block plus the k_i - 1 best earlier blocks,
// k_i = ceil((i + 1) * keep_num / keep_den) (the 90%-sparsity regime of the
// v2 abstract at keep 1/10).
//
// Kernels (gfx950):
//   prefill_pool_project : mean-pool Q and K per block (partial last block:
//                          mean of its rows), one wave per (block, tensor),
//                          then project with Wq / Wk on fp32 MFMA
//   prefill_gate_select  : S_ij = gate_scale * A_i . C_j for 16 query blocks
//                          per workgroup on fp32 MFMA, kept in LDS as order
//                          keys; one wave per row then selects the exact
//                          top-(k_i - 1) of j < i with lower-id ties, then the
//                          diagonal (nb up to 2048)
//   prefill_gate_scores  : beyond 2048 blocks, S into the workspace in fp32
//                          (64x64 tiles through LDS)
//   prefill_select_rows  : beyond 2048 blocks, one wave per row selecting from
//                          the workspace scores by the same rule
//   prefill_attention    : 64 query rows per workgroup; each wave takes 32
//                          rows and one 32-key half of every kept block, MFMA
//                          v_mfma_f32_32x32x16_bf16.  S^T = K Q^T so that each
//                          lane holds one query row's probabilities in exactly
//                          the operand layout of O^T = V^T P^T; K and V tiles
//                          go from HBM straight into double-buffered LDS
//                          (XOR-swizzled against bank conflicts, V^T read with
//                          transposing LDS reads) while the previous block is
//                          computed, and the two key halves of each row are
//                          merged once at the end.
#include "seer_device.hpp"
#include "seer_host.hpp"
#include "topk_wave.hpp"

#include <math.h>
#include <type_traits>

namespace seer {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPBS = 64;  // prefill block size (query and key blocks)
constexpr int kPoolBlocks = 16;  // blocks per workgroup of the gate's pooling kernel
constexpr float kLazyRescale = 8.0f;  // largest log2 weight before the running reference moves

__device__ __forceinline__ int keep_count(int i, int num, int den) {
    const int64_t k = ((int64_t)(i + 1) * num + den - 1) / den;
    return k < 1 ? 1 : (k > i + 1 ? i + 1 : (int)k);
}

__device__ __forceinline__ void unpack8f(const uint4 w, float *f) {
    f[0] = bf16lo(w.x); f[1] = bf16hi(w.x); f[2] = bf16lo(w.y); f[3] = bf16hi(w.y);
    f[4] = bf16lo(w.z); f[5] = bf16hi(w.z); f[6] = bf16lo(w.w); f[7] = bf16hi(w.w);
}

// ---------------------------------------------------------------- gate ----
// Gate rows A_i = Wq qbar_i and C_j = Wk kbar_j are stored fp32 with a row
// stride of DGP = dg rounded up to 128 or 256, zeros past dg, so that the score
// kernels read whole 32-float runs without a tail.
__host__ __device__ constexpr int gate_row_stride(int dg) { return dg <= 128 ? 128 : 256; }

// One workgroup per (chunk of PB blocks, head, batch).  Pooling: the 2 PB
// (block, tensor) items go to the 4 waves round-robin; lane (r4, c) of a wave
// sums rows r4, r4 + 4, ..., r4 + 60 of its item's column chunk c (16 bytes),
// 16 loads in flight per lane, and the four row phases combine across lanes.
// Rows past L read as zero (buffer range), and the mean divides by the rows
// present.  Then the projections run on fp32 MFMA (below).
template <int D>
__global__ __launch_bounds__(256) void prefill_pool_project_kernel(const uint16_t *q, const uint16_t *k, int H,
                                                                   int L, int nb, const uint16_t *wq,
                                                                   const uint16_t *wk, int dg, int dgp, float *A,
                                                                   float *Cm) {
    constexpr int CH = D / 8, PB = kPoolBlocks;
    constexpr int PH = 64 / CH;           // row phases per wave (4)
    constexpr int RPL = kPBS / PH;        // rows per lane and item (16)
    static_assert(D == 128, "one wave covers a 256-byte row in 16 lanes");
    static_assert(PB == 16, "the projection's MFMA columns are the chunk's 16 blocks");
    const int blk0 = blockIdx.x * PB, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    // wave-uniform, so that the Q / K descriptor choice per item stays scalar
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __shared__ float pooled[2][PB][D];  // [Q/K][block][dim]
    const int64_t head = ((int64_t)b * H + h) * L * D;
    const uint32_t bytes = (uint32_t)L * D * 2u;
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(q + head, bytes), rk = buffer_rsrc(k + head, bytes);
    const int nblk = nb - blk0 < PB ? nb - blk0 : PB;
    const int items = 2 * nblk;
    const uint32_t lane_off = (uint32_t)((lane / CH) * D + (lane % CH) * 8) * 2u;
    uint4 cur[RPL];
    for (int it = wave; it < items; it += 4) {
        {  // the whole offset in the per-lane part, which is what the range check covers
            const uint32_t voff = (uint32_t)(blk0 + (it >> 1)) * kPBS * D * 2u + lane_off;
            const __amdgpu_buffer_rsrc_t r = (it & 1) ? rk : rq;
            // each row is read once here: streaming loads keep the pass from
            // evicting what the score and attention kernels reuse
#pragma unroll
            for (int m = 0; m < RPL; ++m) cur[m] = buf_ld16_nt(r, voff + (uint32_t)(m * PH * D * 2), 0);
        }
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < RPL; ++m) {
            float f[8];
            unpack8f(cur[m], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += f[e];
        }
        const int t0 = (blk0 + (it >> 1)) * kPBS;
        const float inv_rows = 1.0f / (float)(L - t0 < kPBS ? L - t0 : kPBS);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = sum_xor32(sum_xor16(acc[e]));
        if (lane < CH) {
#pragma unroll
            for (int e = 0; e < 8; ++e) pooled[it & 1][it >> 1][lane * 8 + e] = acc[e] * inv_rows;
        }
    }
    __syncthreads();
    // A[p][r] = Wq[h][r] . qbar_p ; C[p][r] = Wk[h][r] . kbar_p ; zero for dg <= r < dgp.
    // v_mfma_f32_16x16x4f32 with W rows as M (16-row tiles), the chunk's pooled
    // blocks as N (columns nblk..15 zero) and the D terms split into four contiguous
    // quarters, one per k slot (slot kq carries term kq D/4 + s at step s).  Wave
    // w projects tensor w & 1, row tiles (w >> 1) + 2 m.
    constexpr int QK = D / 4;
    const int n = lane & 15, kq = lane >> 4, t = wave & 1;
    float bop[QK];
#pragma unroll
    for (int s4 = 0; s4 < QK; s4 += 4) {
        const float4 x = n < nblk ? *reinterpret_cast<const float4 *>(&pooled[t][n][kq * QK + s4])
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
        bop[s4] = x.x; bop[s4 + 1] = x.y; bop[s4 + 2] = x.z; bop[s4 + 3] = x.w;
    }
    const uint16_t *w = (t ? wk : wq) + (int64_t)h * dg * D + kq * QK;
    // Results go through LDS, 128 columns at a time, so that the chunk's rows
    // (contiguous in A / C) are written with coalesced 16-byte stores.
    __shared__ __align__(16) float stage[2][PB][128];
    for (int c0 = 0; c0 < dgp; c0 += 128) {
        for (int rt = c0 / 16 + (wave >> 1); rt < c0 / 16 + 8; rt += 2) {
            const int r = rt * 16 + n;
            uint4 wv[QK / 8];
#pragma unroll
            for (int v = 0; v < QK / 8; ++v)
                wv[v] = r < dg ? *reinterpret_cast<const uint4 *>(w + (int64_t)r * D + 8 * v) : make_uint4(0, 0, 0, 0);
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int v = 0; v < QK / 8; ++v) {
                float f[8];
                unpack8f(wv[v], f);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f[e], bop[8 * v + e], acc, 0, 0, 0);
            }
            // rows rt*16 + 4 kq .. + 3 of block n
            *reinterpret_cast<float4 *>(&stage[t][n][rt * 16 - c0 + 4 * kq]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
        __syncthreads();
        for (int x = tid; x < 2 * nblk * 32; x += 256) {  // 32 float4 per block row of the chunk
            const int tt = x / (nblk * 32), p = (x / 32) % nblk, q4 = x % 32;
            float *dst = (tt ? Cm : A) + (((int64_t)b * H + h) * nb + blk0 + p) * dgp + c0 + 4 * q4;
            *reinterpret_cast<float4 *>(dst) = *reinterpret_cast<const float4 *>(&stage[tt][p][4 * q4]);
        }
        __syncthreads();  // the stage is free for the next chunk
    }
}

// The k largest of the n keys of one row in LDS (0 < k < n), ids ascending to
// out, by one wave: the same rule and steps as wave_topk_from_keys (8-bit radix
// passes from the top digit over a 256-bin LDS histogram, then one sweep in id
// order, stopping once the digits so far single out a bin taken whole), with the
// first 64 KR keys held in registers through all passes, so a pass issues its
// histogram atomics back to back instead of after a key read each.
template <int KR>
__device__ __forceinline__ void wave_topk_row(int n, int k, const uint32_t *keys, int *hist, int32_t *out, int lane) {
    uint32_t kreg[KR];
#pragma unroll
    for (int r = 0; r < KR; ++r) kreg[r] = lane + 64 * r < n ? keys[lane + 64 * r] : 0u;
    uint32_t prefix = 0, mask = 0xFFFFFFFFu;  // the digits found so far, and the bits they cover
    int need = k;  // keys still to take among those matching `prefix`
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
#pragma unroll
        for (int i = 0; i < 4; ++i) hist[lane * 4 + i] = 0;
        wave_lds_sync();
#pragma unroll
        for (int r = 0; r < KR; ++r)
            if (lane + 64 * r < n && (kreg[r] & hi_mask) == prefix) atomicAdd(&hist[(kreg[r] >> shift) & 255u], 1);
        for (int j = lane + 64 * KR; j < n; j += 64) {
            const uint32_t key = keys[j];
            if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
        wave_lds_sync();
        // lane l covers digits 255 - 4l .. 252 - 4l, in descending order
        int cnt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cnt[i] = hist[255 - 4 * lane - i];
        const int local = cnt[0] + cnt[1] + cnt[2] + cnt[3];
        const int incl = wave_inclusive_scan(local, lane);
        const int excl = incl - local;
        int digit = 0, rest = 0, whole = 0, cum = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (cum < need && cum + cnt[i] >= need) {  // the digit where the count reaches need
                digit = 255 - 4 * lane - i;
                rest = need - cum;
                whole = rest == cnt[i];
            }
            cum += cnt[i];
        }
        const uint64_t hit = __ballot(excl < need && incl >= need);  // exactly one lane
        const int src = hit ? (int)__builtin_ctzll(hit) : 0;
        prefix |= (uint32_t)__builtin_amdgcn_readlane(digit, src) << shift;
        need = __builtin_amdgcn_readlane(rest, src);
        wave_lds_sync();  // every lane has read the bins before the next pass clears them
        if (__builtin_amdgcn_readlane(whole, src)) {  // a bin taken whole: no further digit matters
            mask = 0xFFFFFFFFu << shift;
            break;
        }
    }
    // keep keys > T and the first `need` keys == T, in id order, on the bits of `mask`
    const uint32_t T = prefix;
    int written = 0, eq_seen = 0;
    for (int base = 0, r = 0; base < n; base += 64, ++r) {
        const int j = base + lane;
        uint32_t key = 0u;
#pragma unroll
        for (int rr = 0; rr < KR; ++rr)
            if (r == rr) key = kreg[rr];
        if (r >= KR) key = j < n ? keys[j] : 0u;
        key &= mask;
        const bool eq = j < n && key == T;
        const uint64_t eq_mask = __ballot(eq);
        const bool take = j < n && (key > T || (eq && eq_seen + lanes_below(eq_mask) < need));
        const uint64_t take_mask = __ballot(take);
        const int pos = written + lanes_below(take_mask);
        if (take && pos < k) out[pos] = j;
        written += __popcll(take_mask);
        eq_seen += __popcll(eq_mask);
    }
}

// Scores and selection of 16 query blocks i0 .. i0 + 15 of one (b, h) per
// workgroup, for nb <= kGsMaxCols.  The 16 x 16 score tiles of key blocks
// 16 t .. 16 t + 15, t <= the group's own tile, go to the waves round-robin and
// run on v_mfma_f32_16x16x4f32 (A operand: lane (kq, n) holds row n, k slot kq;
// B: k slot kq, column n; result: rows 4 kq + e, column n).  The dot product
// over DGP terms is split into four contiguous quarters, one per k slot: at
// step s, slot kq carries term kq DGP / 4 + s, so each lane reads its row's and
// its column's quarter as 16-byte loads straight from the gate rows.  Scores,
// times gate_scale, are kept in LDS as order keys; then wave w selects rows
// w, w + 4, w + 8, w + 12 (exact top-(k_i - 1) of j < i, lower id on ties,
// ascending, then the diagonal i).  The heaviest row groups (the last) start first.
constexpr int kGsRows = 16;
constexpr int kGsMaxCols = 2048;

__host__ __device__ constexpr int gs_key_stride(int nb) { return (nb + 15) / 16 * 16 + 4; }

template <int DGP>
__global__ __launch_bounds__(256) void prefill_gate_select_kernel(const float *A, const float *Cm, int BH, int nb,
                                                                  float gate_scale, int keep_num, int keep_den,
                                                                  int kmax_row, int32_t *kv_blocks,
                                                                  int32_t *kv_count) {
    constexpr int QK = DGP / 4;        // terms per k slot
    constexpr int NV = QK / 4;         // 16-byte loads per lane and operand
    extern __shared__ uint32_t gs_lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nrg = (nb + kGsRows - 1) / kGsRows;
    const int rgi = nrg - 1 - (int)(blockIdx.x / BH), bh = (int)(blockIdx.x % BH);
    const int i0 = rgi * kGsRows;
    const int ks = gs_key_stride(nb);
    uint32_t *keys = gs_lds;                                   // [16][ks]
    int *hist = reinterpret_cast<int *>(gs_lds + kGsRows * ks) + wave * 256;
    const int n = lane & 15, kq = lane >> 4;
    const float *Ab = A + (int64_t)bh * nb * DGP, *Cb = Cm + (int64_t)bh * nb * DGP;
    // this lane's query row (clamped: rows past nb are never selected for)
    const int ia = i0 + n < nb ? i0 + n : nb - 1;
    float4 av[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) av[v] = *reinterpret_cast<const float4 *>(Ab + (int64_t)ia * DGP + kq * QK + 4 * v);
    const int ntile = rgi + 1;  // key tiles 0 .. rgi
    float4 cv[NV], cn[NV];
    auto load_c = [&](float4 (&buf)[NV], int t) {
        const int j = 16 * t + n < nb ? 16 * t + n : nb - 1;
#pragma unroll
        for (int v = 0; v < NV; ++v) buf[v] = *reinterpret_cast<const float4 *>(Cb + (int64_t)j * DGP + kq * QK + 4 * v);
    };
    load_c(cv, wave < ntile ? wave : 0);
    for (int t = wave; t < ntile; t += 4) {
        load_c(cn, t + 4 < ntile ? t + 4 : t);  // unconditional (a cached re-read at the end): see the pooling loop
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[v].x, cv[v].x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[v].y, cv[v].y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[v].z, cv[v].z, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[v].w, cv[v].w, acc, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) keys[(4 * kq + e) * ks + 16 * t + n] = order_key(acc[e] * gate_scale);
#pragma unroll
        for (int v = 0; v < NV; ++v) cv[v] = cn[v];
    }
    __syncthreads();
    for (int rr = wave; rr < kGsRows; rr += 4) {
        const int i = i0 + rr;
        if (i >= nb) break;
        const int64_t row = (int64_t)bh * nb + i;
        int32_t *out = kv_blocks + row * kmax_row;
        int ki = keep_count(i, keep_num, keep_den);
        ki = ki > kmax_row ? kmax_row : ki;
        const int need = ki - 1;
        if (need > 0 && need < i) {
            wave_topk_row<8>(i, need, keys + rr * ks, hist, out, lane);
        } else if (need > 0) {  // every earlier block is kept
            for (int m = lane; m < need; m += 64) out[m] = m;
        }
        for (int m = need + lane; m < kmax_row; m += 64) out[m] = m == need ? i : -1;
        if (lane == 0) kv_count[row] = need + 1;
        wave_lds_sync();  // the next row's passes reuse hist
    }
}

// S[b][h][i][j] = gate_scale * A_i . C_j for the lower-triangular 64x64 tiles.
// One workgroup per (row tile, column tile <= row tile, head*batch).
__global__ __launch_bounds__(256) void prefill_gate_scores_kernel(const float *A, const float *Cm, int nb, int dg,
                                                                  float gate_scale, float *S) {
    constexpr int T = 64, KC = 32;
    const int it = blockIdx.x, jt = blockIdx.y, bh = blockIdx.z;
    if (jt > it) return;
    __shared__ float as[KC][T + 1], cs[KC][T + 1];
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
    const float *Ab = A + (int64_t)bh * nb * dg, *Cb = Cm + (int64_t)bh * nb * dg;
    float acc[4][4] = {};
    for (int e0 = 0; e0 < dg; e0 += KC) {
        for (int x = tid; x < T * KC; x += 256) {
            const int r = x / KC, e = x % KC;
            const int ri = it * T + r, rj = jt * T + r;
            as[e][r] = (ri < nb && e0 + e < dg) ? Ab[(int64_t)ri * dg + e0 + e] : 0.f;
            cs[e][r] = (rj < nb && e0 + e < dg) ? Cb[(int64_t)rj * dg + e0 + e] : 0.f;
        }
        __syncthreads();
#pragma unroll 8
        for (int e = 0; e < KC; ++e) {
            float a[4], cc[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                a[u] = as[e][ty * 4 + u];
                cc[u] = cs[e][tx * 4 + u];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a[u], cc[v], acc[u][v]);
        }
        __syncthreads();
    }
    float *Sb = S + (int64_t)bh * nb * nb;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = it * T + ty * 4 + u;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int j = jt * T + tx * 4 + v;
            if (i < nb && j < nb && j <= i) Sb[(int64_t)i * nb + j] = acc[u][v] * gate_scale;
        }
    }
}

// Row i keeps the best k_i - 1 blocks j < i (lower id on ties), ascending, then i.
__global__ __launch_bounds__(256) void prefill_select_rows_kernel(const float *S, int BH, int nb, int slice,
                                                                  int keep_num, int keep_den, int kmax_row,
                                                                  int32_t *kv_blocks, int32_t *kv_count) {
    extern __shared__ uint32_t lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;  // bh * nb + i
    if (row >= (int64_t)BH * nb) return;
    const int i = (int)(row % nb);
    uint32_t *keys = lds + (size_t)wave * slice;
    int *hist = reinterpret_cast<int *>(keys + slice - 256);
    int32_t *out = kv_blocks + row * kmax_row;
    int ki = keep_count(i, keep_num, keep_den);
    ki = ki > kmax_row ? kmax_row : ki;
    const int need = ki - 1;
    if (need > 0 && need < i) {
        wave_topk_ascending<LaunchMem>(S + row * nb, i, need, keys, hist, out, lane);
    } else if (need > 0) {  // every earlier block is kept
        for (int m = lane; m < need; m += 64) out[m] = m;
    }
    wave_lds_sync();
    for (int m = need + lane; m < kmax_row; m += 64) out[m] = m == need ? i : -1;
    if (lane == 0) kv_count[row] = need + 1;
}

// ----------------------------------------------------------- attention ----
// Workgroup of 4 waves per 64-row query block.  Wave w owns query rows
// 32 (w & 1) + 0..31 and keys 32 (w >> 1) + 0..31 of every kept key block, so
// each K / V element staged in LDS is read by two waves instead of four; the
// two key halves of a row are merged once at the end (their running maxima and
// sums combine as in split-KV decoding).
//
// Both products run on v_mfma_f32_32x32x16_bf16, which this part sustains at
// about twice the rate of the 16x16x32 shape:
//   S^T = K Q^T   A = 32 keys x 16 dims (one 16-byte K chunk per lane), B = Q^T
//                 held in registers.  Lane l ends with query row l % 32 and the
//                 wave's keys 8 a + 4 hl + b (a, b = 0..3, hl = l / 32).
//   O^T = V^T P^T B = P^T: k-step s takes the lane's own keys with a = 2 s and
//                 2 s + 1, so the weights never move between lanes; A = V^T, two
//                 ds_read_b64_tr_b16 per lane from the 4-key groups 16 s + 4 hl
//                 (k slots 8 hl + 0..3) and 16 s + 8 + 4 hl (slots 8 hl + 4..7),
//                 exactly those keys.
//   A query row's statistics live in two lanes (l and l ^ 32): one swap each.
//
// LDS layouts (one 64-key block of 256-byte rows).  buffer_load ... lds writes
// lane l's 16 bytes at the wave's LDS base + 16 l, so a swizzle is a choice of
// which global chunk each lane loads.
//  K : 16-byte chunk c of key r at slot c ^ (r & 15): an A operand read (32
//      keys, one chunk) hits distinct banks in each 16-lane phase.
//  V : 32-byte chunk c of key r at chunk c ^ 2 (r & 3): a transposing read
//      covers 4 consecutive keys x 2 adjacent chunks per 32 lanes, which land in
//      8 distinct chunks.

// GT (the ground-truth form): every causal block j <= i is attended (the lists
// are not read), and after the output a second sweep over K recomputes the
// scores and writes mass[b][h][i][j] = mean over block i's rows of the weight
// they give block j (zero for j > i).
template <int D, bool GT = false>
__global__ __launch_bounds__(256, 2) void prefill_attention_kernel(const uint16_t *q, const uint16_t *k,
                                                                   const uint16_t *v, int H, int L, int nb,
                                                                   const int32_t *kv_blocks,
                                                                   const int32_t *kv_count, int kmax_row,
                                                                   float scale_log2, uint16_t *out, float *lse,
                                                                   float *mass) {
    static_assert(D == 128, "the LDS layouts assume 256-byte key rows");
    typedef float f32x16_t __attribute__((ext_vector_type(16)));
    typedef short v4s __attribute__((ext_vector_type(4)));
    constexpr int KS = D / 16;           // k-steps of S^T = K Q^T
    constexpr int DT = D / 32;           // 32-wide d tiles of O^T
    constexpr int KBYTES = kPBS * D * 2;
    constexpr int DMA_PER_WAVE = KBYTES / 1024 / 4;  // 1 KiB buffer_load ... lds per wave and tensor
    // Two K and two V buffers (separate objects, so that the compiler sees a load
    // into one buffer does not alias reads of another); the key-half exchange
    // (DT x 16 floats per lane of a row half) reuses the K buffers after the sweep.
    __shared__ __align__(16) char kbuf0[KBYTES], kbuf1[KBYTES], vbuf0[KBYTES], vbuf1[KBYTES];
    __shared__ float xml[2][2][64];   // [rh][m | l][lane] of the key-half-1 waves
    static_assert(DT * 16 * 64 * 4 <= KBYTES, "one row half's exchange fits a K buffer");

    // Workgroups reach the 8 XCDs round-robin (id % 8); give each XCD one
    // contiguous range of the (b, h)-major list so that a head's K / V blocks
    // are fetched into one L2 instead of all eight.  Longest rows first: within
    // each (b, h) the last query block comes first.
    const int64_t nwg = gridDim.x, xcd = blockIdx.x % 8, local = blockIdx.x / 8;
    const int64_t wi = xcd * (nwg / 8) + (xcd < nwg % 8 ? xcd : nwg % 8) + local;
    const int64_t per_b = (int64_t)H * nb;
    const int b = (int)(wi / per_b);
    const int rem = (int)(wi % per_b);
    const int h = rem / nb;
    const int i = nb - 1 - rem % nb;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rh = wave & 1, kh = wave >> 1;
    const int hl = lane >> 5, n = lane & 31;
    const int64_t head = ((int64_t)b * H + h) * L * D;
    const uint16_t *qh = q + head, *kh_ptr = k + head, *vh = v + head;
    const int qtok = i * kPBS + 32 * rh + n;  // this lane's query row

    // B operand of S^T: lane (hl, n) holds dims 16 ks + 8 hl .. + 7 of query row qtok.
    bf16x8_t qop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const uint4 w = qtok < L ? *reinterpret_cast<const uint4 *>(qh + (int64_t)qtok * D + 16 * ks + 8 * hl)
                                 : make_uint4(0, 0, 0, 0);
        qop[ks] = __builtin_bit_cast(bf16x8_t, w);
    }
    f32x16_t oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f, m_ref = 0.f;

    const int64_t row = ((int64_t)b * H + h) * nb + i;
    int cnt = GT ? i + 1 : kv_count[row];
    cnt = cnt < 0 ? 0 : (cnt > kmax_row ? kmax_row : cnt);
    // The lists are read-only here: read them through the constant address
    // space so that they are scalar loads, which do not wait behind the
    // in-flight K / V loads the way a vector load's vmcnt would.
    typedef const __attribute__((address_space(4))) int32_t const_i32;
    const_i32 *blist = GT ? nullptr : (const_i32 *)(kv_blocks + row * kmax_row);
    auto block_of = [&](int it) { return GT ? it : blist[it]; };

    // K and V of the head through buffer descriptors, loaded straight into LDS.
    // Wave w fills rows 16w..16w+15 of a buffer, 4 rows (1 KiB) per load; lane
    // l takes row 16w + 4q + l / 16 and the global chunk whose swizzled slot is
    // l % 16.  In the last block of a context that is not a multiple of 64,
    // rows past the end read the last token (their scores are masked).
    const uint32_t head_bytes = (uint32_t)((int64_t)L * D * 2);
    const auto krs = buffer_rsrc(kh_ptr, head_bytes), vrs = buffer_rsrc(vh, head_bytes);
    uint32_t kdv[DMA_PER_WAVE], vdv[DMA_PER_WAVE];
    int drow[DMA_PER_WAVE];
#pragma unroll
    for (int qd = 0; qd < DMA_PER_WAVE; ++qd) {
        const int r = 16 * wave + 4 * qd + (lane >> 4), s = lane & 15;
        drow[qd] = r;
        kdv[qd] = (uint32_t)(r * D * 2 + ((s ^ (r & 15)) << 4));
        vdv[qd] = (uint32_t)(r * D * 2 + (((((s >> 1) ^ (2 * (r & 3))) << 1) | (s & 1)) << 4));
    }
    auto block_start = [&](int it) {
        int j = block_of(it);
        j = j < 0 ? 0 : (j > i ? i : j);
        return j * kPBS;
    };
    auto dma_at = [&](int k0, char *dst, __amdgpu_buffer_rsrc_t rs, const uint32_t (&dv)[DMA_PER_WAVE]) {
        char *base = dst + wave * (DMA_PER_WAVE * 1024);
        if (k0 + kPBS <= L) {  // a whole block: the row offset is scalar
#pragma unroll
            for (int qd = 0; qd < DMA_PER_WAVE; ++qd)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(base + qd * 1024),
                                                         16, (int)dv[qd], k0 * D * 2, 0, 0);
        } else {  // the context's partial last block
#pragma unroll
            for (int qd = 0; qd < DMA_PER_WAVE; ++qd) {
                const int over = drow[qd] - (L - 1 - k0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(base + qd * 1024),
                                                         16, (int)dv[qd] - (over > 0 ? over : 0) * D * 2, k0 * D * 2, 0, 0);
            }
        }
    };
    auto dma = [&](int it, char *dst, __amdgpu_buffer_rsrc_t rs, const uint32_t (&dv)[DMA_PER_WAVE]) {
        dma_at(block_start(it), dst, rs, dv);
    };
    auto loads_done = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0): this wave's loads are in LDS
    // S^T of this wave's 32 keys and 32 query rows: s[4 a + b] holds key
    // 32 kh + 8 a + 4 hl + b of query row qtok.  One accumulation chain over
    // the 8 k-steps: the P V products of the previous block fill the gaps
    // between its dependent MFMAs, and no VALU adds of partial sums remain.
    // kread: the K operand of this wave's 32 keys for every k-step (offsets masked
    // to the buffer's 16 KiB, which they never exceed: the compiler then sees that
    // the reads cannot touch a buffer being loaded).  smma: the MFMAs.
    const int krow_off = (32 * kh + n) * (D * 2);
    auto kread = [&](bf16x8_t (&ka)[KS], const char *kb) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            ka[ks] = *reinterpret_cast<const bf16x8_t *>(
                kb + ((krow_off + (((2 * ks + hl) ^ (n & 15)) << 4)) & (KBYTES - 1)));
    };
    auto smma = [&](f32x16_t &s, const bf16x8_t (&ka)[KS]) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qop[ks], s, 0, 0, 0);
    };
    auto scores = [&](f32x16_t &s, const char *kb) {
        bf16x8_t ka[KS];
        kread(ka, kb);
        smma(s, ka);
    };
    // Causal / length masks: only the diagonal block and a partial last block need them.
    auto edge_at = [&](int k0) { return k0 == i * kPBS || k0 + kPBS > L; };
    auto mask_at = [&](f32x16_t &s, int k0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int ktok = k0 + 32 * kh + 8 * (e >> 2) + 4 * hl + (e & 3);
            if (ktok > qtok || ktok >= L) s[e] = -INFINITY;
        }
    };
    // Running maximum with lazy rescaling: the reference m_run moves only when
    // the block's maximum exceeds it by more than kLazyRescale (log2 units), so
    // the weights stay below 2^kLazyRescale and O is rarely rescaled.  Any
    // reference gives the same softmax once O is divided by l.  m_ref is m_run,
    // or 0 while that is -inf.  Each lane first tests its own scores: rounding
    // is monotone, so some lane's max * scale exceeds the bound exactly when the
    // row's max * scale does, and the partner exchange and the rescale run only
    // in the (rare) blocks where a reference moves.
    auto prep = [&](const f32x16_t &s, bool live) {
        float lmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) lmax = fmax_fast(lmax, s[e]);
        const bool need = live && lmax * scale_log2 > m_run + kLazyRescale;  // always when m_run is still -inf
        if (!__ballot(need)) return;
        const float mloc = max_xor32(lmax) * scale_log2;  // the two lanes of this query row
        const bool bump = live && mloc > m_run + kLazyRescale;
        const float m_new = bump ? mloc : m_run;
        const float ref = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = bump ? fast_exp2(m_run - ref) : 1.0f;
        m_run = m_new;
        m_ref = ref;
        if (__ballot(bump)) {  // some row's reference moved
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
            l_run *= alpha;
        }
    };
    // Weights of one block (relative to m_ref) into the P^T operands of the two
    // k-steps: pb[s] = weights s[8 s .. 8 s + 7].
    auto weights = [&](f32x16_t &s, bf16x8_t (&pb)[2]) {
        float lsum = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float p = fast_exp2(fmaf(s[e], scale_log2, -m_ref));
            s[e] = p;
            lsum += p;
        }
        l_run += lsum;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pb[0][e] = (__bf16)s[e];
            pb[1][e] = (__bf16)s[8 + e];
        }
    };
    // V^T operand of d tile dt and k-step s: lane (hl, dg, j) (j = lane % 16,
    // dg = lane / 16 % 2) points at key 32 kh + 16 s + 4 hl + j / 4 (and + 8),
    // columns 32 dt + 16 dg + 4 (j % 4) + 0..3; after the transpose it holds
    // column 32 dt + 16 dg + j of 4 keys.  The key's swizzle 2 (r & 3) is
    // 2 (j / 4) for every such key.
    // The byte offset within the tile takes only the bits of rows 0..7 and
    // 32..39 (0x2000, 0x0700) and of the chunk and column terms (0x00F8).  Masking
    // it with exactly those bits changes nothing, but lets the compiler see that
    // the reads stay inside this V buffer: otherwise it cannot rule out the
    // in-flight loads into the other buffers and waits for them (vmcnt(0)) in
    // the middle of every iteration.
    const int tj = lane & 15, tdg = (lane >> 4) & 1;
    const int vrow_rd = 32 * kh + 4 * hl + (tj >> 2);
    constexpr int kVReadBits = 0x2000 | 0x0700 | 0x00F8;
    auto pv = [&](const bf16x8_t (&pb)[2], const char *vb) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const char *pcol =
                vb + ((vrow_rd * (D * 2) + ((dt ^ (tj >> 2)) << 6) + (tdg << 5) + ((tj & 3) << 3)) & kVReadBits);
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const char *p = pcol + 16 * st * (D * 2);
                const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)p);
                const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4s *)(p + 8 * D * 2));
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st], oacc[dt], 0, 0, 0);
            }
        }
    };

    // Software pipeline over double-buffered LDS.  Iteration it computes the
    // scores of block it + 1 and P V of block it (MFMA) alongside the weights of
    // block it (VALU), then masks block it + 1 if it is an edge block and takes
    // its maximum.  At its start it issues the loads of K of block it + 2 and V
    // of block it + 1 into the buffers the last iteration finished with; they
    // land while it computes.  One barrier per iteration.  Buffer parity follows
    // it, so the loop is unrolled by two.  The first tokens of blocks it + 1 and
    // it + 2 are carried from iteration to iteration, so each reads one block id
    // (block it + 3's) and before it is needed.
    f32x16_t sA, sB;
    int kn1 = 0, kn2 = 0;
    if (cnt > 0) {
        const int k0 = block_start(0);
        kn1 = cnt > 1 ? block_start(1) : 0;
        kn2 = cnt > 2 ? block_start(2) : 0;
        dma_at(k0, kbuf0, krs, kdv);
        dma_at(k0, vbuf0, vrs, vdv);
        if (cnt > 1) dma_at(kn1, kbuf1, krs, kdv);
        loads_done();
        __syncthreads();
        scores(sA, kbuf0);
        if (edge_at(k0)) mask_at(sA, k0);
        prep(sA, true);
        __syncthreads();  // block 0's K buffer is free
    }
    // s_cur holds block it's masked scores with its reference applied to O and
    // l; s_next receives block it + 1.  P = it & 1 (compile-time).
    auto step = [&](auto par, int it, f32x16_t &s_cur, f32x16_t &s_next) {
        constexpr int P = decltype(par)::value;
        char *const k_this = P ? kbuf1 : kbuf0, *const k_next = P ? kbuf0 : kbuf1;
        char *const v_this = P ? vbuf1 : vbuf0, *const v_next = P ? vbuf0 : vbuf1;
        const bool has_next = it + 1 < cnt;
        if (it + 2 < cnt) dma_at(kn2, k_this, krs, kdv);  // where block it's K was
        if (has_next) dma_at(kn1, v_next, vrs, vdv);       // where block it - 1's V was
        const int k1 = kn1;
        const int kn3 = it + 3 < cnt ? block_start(it + 3) : 0;
        // One straight-line region (no branch inside) so that the MFMAs of the
        // scores and of P V interleave with the VALU work on the weights.
        bf16x8_t pb[2];
        scores(s_next, k_next);  // on the last step this reads a stale buffer: unused
        weights(s_cur, pb);
        pv(pb, v_this);
        if (has_next && edge_at(k1)) mask_at(s_next, k1);
        prep(s_next, has_next);
        kn1 = kn2;
        kn2 = kn3;
        loads_done();
        __syncthreads();  // loads visible; reads of this iteration's buffers done
    };
    for (int it = 0; it < cnt; it += 2) {
        step(std::integral_constant<int, 0>{}, it, sA, sB);
        if (it + 1 >= cnt) break;
        step(std::integral_constant<int, 1>{}, it + 1, sB, sA);
    }

    // Merge the two key halves of each row: the kh = 1 waves hand (m, l, O) to
    // their kh = 0 partners through LDS.
    const float l_row = sum_xor32(l_run);
    float *xo = reinterpret_cast<float *>(rh ? kbuf1 : kbuf0);  // per row half: [dt][e4][lane][4] floats
    __syncthreads();  // the staging area is free
    if (kh == 1) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
                *reinterpret_cast<f32x4_t *>(xo + ((dt * 4 + e4) * 64 + lane) * 4) =
                    f32x4_t{oacc[dt][4 * e4], oacc[dt][4 * e4 + 1], oacc[dt][4 * e4 + 2], oacc[dt][4 * e4 + 3]};
        xml[rh][0][lane] = m_run;
        xml[rh][1][lane] = l_row;
    }
    __syncthreads();
    float lse2 = 0.f;  // final log2-domain row log-sum-exp (kh = 0 waves)
    if (kh == 0) {
        const float m1 = xml[rh][0][lane], l1 = xml[rh][1][lane];
        const float m = fmax_fast(m_run, m1);
        const float mr = m == -INFINITY ? 0.f : m;
        const float a0 = fast_exp2(m_run - mr), a1 = fast_exp2(m1 - mr);
        const float l_tot = l_row * a0 + l1 * a1;
        lse2 = l_tot > 0.f ? m + log2f(l_tot) : INFINITY;
        if (qtok < L) {
            const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
            uint16_t *orow = out + head + (int64_t)qtok * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {  // d = 32 dt + 8 e4 + 4 hl + 0..3
                    const f32x4_t o1 = *reinterpret_cast<const f32x4_t *>(xo + ((dt * 4 + e4) * 64 + lane) * 4);
                    const f32x4_t o0 = f32x4_t{oacc[dt][4 * e4], oacc[dt][4 * e4 + 1], oacc[dt][4 * e4 + 2],
                                               oacc[dt][4 * e4 + 3]};
                    const f32x4_t o = (o0 * a0 + o1 * a1) * inv;
                    const uint32_t w0 = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
                    const uint32_t w1 = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
                    *reinterpret_cast<uint2 *>(orow + 32 * dt + 8 * e4 + 4 * hl) = make_uint2(w0, w1);
                }
            if (hl == 0 && lse) lse[((int64_t)b * H + h) * L + qtok] = l_tot > 0.f ? lse2 * kLn2 : -INFINITY;
        }
    }
    if constexpr (GT) {
        // Second sweep: each block's share of every row's softmax, averaged over
        // the block's rows.  The K tiles rotate through all four tile buffers,
        // three blocks ahead of the one being scored, with one barrier per block;
        // the block's sum over the four waves goes through a double-buffered slot
        // and is written out by thread 0 after the next barrier.
        __shared__ float row_lse2[64];
        __shared__ float red[2][4];
        if (kh == 0 && hl == 0) row_lse2[32 * rh + n] = lse2;
        __syncthreads();  // also: the exchange area in the K buffers is free
        lse2 = row_lse2[32 * rh + n];
        const int rows_i = L - i * kPBS < kPBS ? L - i * kPBS : kPBS;
        float *mrow = mass + row * nb;
        for (int jj = i + 1 + tid; jj < nb; jj += 256) mrow[jj] = 0.f;
        auto block_mass_out = [&](int jb) {
            if (tid == 0) mrow[jb] = (red[jb & 1][0] + red[jb & 1][1] + red[jb & 1][2] + red[jb & 1][3]) / (float)rows_i;
        };
        dma(0, kbuf0, krs, kdv);
        if (i >= 1) dma(1, kbuf1, krs, kdv);
        if (i >= 2) dma(2, vbuf0, krs, kdv);
        auto sweep = [&](auto par, int jb) {
            constexpr int P = decltype(par)::value;
            char *const cur = P == 0 ? kbuf0 : (P == 1 ? kbuf1 : (P == 2 ? vbuf0 : vbuf1));
            char *const nxt3 = P == 0 ? vbuf1 : (P == 1 ? kbuf0 : (P == 2 ? kbuf1 : vbuf0));  // block jb - 1's
            // This wave's loads of block jb have landed once at most its loads of
            // the later blocks (up to two) are still in flight; then a plain
            // s_barrier (a __syncthreads would wait for those too).
            const int later = i - jb < 2 ? i - jb : 2;
            if (later == 2)
                __builtin_amdgcn_s_waitcnt((2 * DMA_PER_WAVE) | 0x0070);  // vmcnt(8), lgkmcnt(0)
            else if (later == 1)
                __builtin_amdgcn_s_waitcnt(DMA_PER_WAVE | 0x0070);
            else
                __builtin_amdgcn_s_waitcnt(0x0070);
            __asm__ volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            __asm__ volatile("" ::: "memory");
            if (jb > 0) block_mass_out(jb - 1);
            bf16x8_t ka[KS];
            kread(ka, cur);
            if (jb + 3 <= i) dma(jb + 3, nxt3, krs, kdv);  // after this block's K reads
            f32x16_t s;
            smma(s, ka);
            const int k0 = jb * kPBS;
            float psum = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int ktok = k0 + 32 * kh + 8 * (e >> 2) + 4 * hl + (e & 3);
                const bool live = ktok <= qtok && ktok < L && qtok < L;
                psum += live ? fast_exp2(s[e] * scale_log2 - lse2) : 0.f;
            }
            psum = wave_sum(psum);
            if (lane == 0) red[jb & 1][wave] = psum;
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        for (int jb = 0; jb <= i; jb += 4) {
            sweep(I0{}, jb);
            if (jb + 1 > i) break;
            sweep(I1{}, jb + 1);
            if (jb + 2 > i) break;
            sweep(I2{}, jb + 2);
            if (jb + 3 > i) break;
            sweep(I3{}, jb + 3);
        }
        __builtin_amdgcn_s_waitcnt(0x0070);
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        block_mass_out(i);
    }
}

}  // namespace seer

using namespace seer;

static int prefill_kmax_row(int nb, int num, int den) {
    int64_t k = ((int64_t)nb * num + den - 1) / den;
    return (int)(k < 1 ? 1 : (k > nb ? nb : k));
}

extern "C" int seer_block_sparse_prefill_kmax_row(int L, int block_size, int keep_num, int keep_den) {
    if (L <= 0 || block_size <= 0 || keep_num < 0 || keep_den <= 0) return 0;
    return prefill_kmax_row((L + block_size - 1) / block_size, keep_num, keep_den);
}

extern "C" size_t seer_block_sparse_prefill_workspace_size(int B, int H, int L, int d, int block_size, int dg) {
    if (B <= 0 || H <= 0 || L <= 0 || d <= 0 || block_size <= 0 || dg <= 0) return 0;
    const size_t nb = (size_t)(L + block_size - 1) / block_size;
    const size_t bh = (size_t)B * H;
    // gate rows A and C; the score matrix only where the fused gate kernel's
    // LDS cannot hold 16 rows of keys
    const size_t scores = nb > (size_t)kGsMaxCols ? bh * nb * nb : 0;
    return (2 * bh * nb * gate_row_stride(dg) + scores) * sizeof(float);
}

extern "C" int seer_block_sparse_prefill(const seer_bf16 *q, const seer_bf16 *k, const seer_bf16 *v, int B, int H,
                                         int L, int d, int block_size, const seer_bf16 *wq, const seer_bf16 *wk,
                                         int dg, float gate_scale, int keep_num, int keep_den, int32_t *kv_blocks,
                                         int32_t *kv_count, int kmax_row, int use_given_blocks, float softmax_scale,
                                         void *workspace, size_t workspace_bytes, seer_bf16 *out, float *lse,
                                         hipStream_t stream) {
    if (!q || !k || !v || !kv_blocks || !kv_count || !out) return SEER_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || L <= 0 || kmax_row <= 0 || !softmax_scale_ok(softmax_scale)) return SEER_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return SEER_ERR_INVALID_ARG;
    if (d != 128 || block_size != kPBS) return SEER_ERR_UNSUPPORTED;
    const int nb = (L + kPBS - 1) / kPBS;
    const int64_t rows = (int64_t)B * H * nb;
    if (rows > 0x7fffffffLL || (int64_t)B * H > 65535) return SEER_ERR_INVALID_ARG;
    if (!use_given_blocks) {
        if (!wq || !wk || dg < 1 || dg > 256 || keep_num < 0 || keep_den <= 0 || !(gate_scale == gate_scale) ||
            !aligned16(wq) || !aligned16(wk))
            return SEER_ERR_INVALID_ARG;
        if (kmax_row < prefill_kmax_row(nb, keep_num, keep_den)) return SEER_ERR_INVALID_ARG;
        if (nb > 16384 - 256) return SEER_ERR_UNSUPPORTED;
        const size_t need = seer_block_sparse_prefill_workspace_size(B, H, L, d, kPBS, dg);
        if (!workspace || workspace_bytes < need || !aligned16(workspace)) return SEER_ERR_WORKSPACE;
        const int dgp = gate_row_stride(dg);
        float *A = static_cast<float *>(workspace);
        float *Cm = A + (size_t)B * H * nb * dgp;
        const dim3 pool_grid((nb + kPoolBlocks - 1) / kPoolBlocks, H, B);
        prefill_pool_project_kernel<128><<<pool_grid, 256, 0, stream>>>(q, k, H, L, nb, wq, wk, dg, dgp, A, Cm);
        int st = launch_status();
        if (st != SEER_OK) return st;
        if (nb <= kGsMaxCols) {
            const int nrg = (nb + kGsRows - 1) / kGsRows;
            const size_t lds = ((size_t)kGsRows * gs_key_stride(nb) + 4 * 256) * sizeof(uint32_t);
            auto kernel = dgp == 128 ? prefill_gate_select_kernel<128> : prefill_gate_select_kernel<256>;
            if (lds > 65536 &&
                hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
                    hipSuccess)
                return SEER_ERR_LAUNCH;
            kernel<<<dim3((unsigned)(nrg * B * H)), 256, lds, stream>>>(A, Cm, B * H, nb, gate_scale, keep_num,
                                                                         keep_den, kmax_row, kv_blocks, kv_count);
            if ((st = launch_status()) != SEER_OK) return st;
        } else {
            float *S = Cm + (size_t)B * H * nb * dgp;
            const int nt = (nb + 63) / 64;
            prefill_gate_scores_kernel<<<dim3(nt, nt, B * H), 256, 0, stream>>>(A, Cm, nb, dgp, gate_scale, S);
            if ((st = launch_status()) != SEER_OK) return st;
            const int slice = nb + 256;
            int waves = (int)(65536 / ((size_t)slice * 4));
            waves = waves < 1 ? 1 : (waves > 4 ? 4 : waves);
            prefill_select_rows_kernel<<<dim3((unsigned)((rows + waves - 1) / waves)), 64 * waves,
                                         (size_t)waves * slice * sizeof(uint32_t), stream>>>(
                S, B * H, nb, slice, keep_num, keep_den, kmax_row, kv_blocks, kv_count);
            if ((st = launch_status()) != SEER_OK) return st;
        }
    }
    prefill_attention_kernel<128><<<dim3((unsigned)rows), 256, 0, stream>>>(
        q, k, v, H, L, nb, kv_blocks, kv_count, kmax_row, softmax_scale * kLog2e, out, lse, nullptr);
    return launch_status();
}

extern "C" int seer_prefill_block_mass(const seer_bf16 *q, const seer_bf16 *k, const seer_bf16 *v, int B, int H,
                                       int L, int d, int block_size, float softmax_scale, seer_bf16 *out, float *lse,
                                       float *mass, hipStream_t stream) {
    if (!q || !k || !v || !out || !mass) return SEER_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || L <= 0 || !softmax_scale_ok(softmax_scale)) return SEER_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return SEER_ERR_INVALID_ARG;
    if (d != 128 || block_size != kPBS) return SEER_ERR_UNSUPPORTED;
    const int nb = (L + kPBS - 1) / kPBS;
    const int64_t rows = (int64_t)B * H * nb;
    if (rows > 0x7fffffffLL) return SEER_ERR_INVALID_ARG;
    prefill_attention_kernel<128, true><<<dim3((unsigned)rows), 256, 0, stream>>>(
        q, k, v, H, L, nb, nullptr, nullptr, nb, softmax_scale * kLog2e, out, lse, mass);
    return launch_status();
}
