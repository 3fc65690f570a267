/*
 * seer_oracle.h -- plain fp64 CPU oracle for gated block-sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP library, and the HIP library never
 * calls it: the two meet only through the seeded input generator and the
 * comparisons in the tests.
 *
 * What it computes (sources: "SeerAttention-R: Sparse Attention Adaptation
 * for Long Reasoning", abstract; "SeerAttention: Learning Intrinsic Sparse
 * Attention in Your LLMs", abstract v1 and v2):
 *
 *   decode, per sequence b and KV head g with group of G query heads
 *     D1  kp_j  = mean of the bs keys of complete block j
 *     D2  s_hj  = (Wq q_h) . (Wk kp_j) * gate_scale   (un-pooled query)
 *     D3  S_j   = mean over the group's query heads of s_hj
 *     D4  keep the k = min(budget / bs, nc) blocks of largest S_j,
 *         ties toward the lower block index, emitted in ascending order
 *     D5  token set T = kept blocks plus the incomplete tail [nc*bs, L)
 *     D6  softmax attention of every query head over T
 *     V1  variant: every query head selects its own blocks by its own s_hj
 *     G1  ground truth: attention mass of every block under dense attention,
 *         averaged over the group's query heads
 *   prefill, per head
 *     P1  mean-pool Q and K over each bs-token block
 *     P2  S_ij = (Wq Qbar_i) . (Wk Kbar_j) * gate_scale for j <= i
 *     P3  row i keeps itself plus the k_i - 1 best earlier blocks,
 *         k_i = ceil((i + 1) * keep_num / keep_den)
 *     P4  causal softmax attention restricted to the kept blocks
 *     G2  ground truth: mean attention mass of every key block per query block
 *
 * All floating point is double.  Inputs arrive as raw bf16 bit patterns
 * (uint16) and are widened exactly.  Strides are in elements.  Every
 * function returns 0 on success and a negative value on a violated
 * precondition, in which case its outputs are unspecified.
 *
 * Parity pins: every function is checked in the CPU tests against closed
 * forms, brute force or a library routine; the choice of gate form, pooling
 * operator and GQA aggregation itself has no page-printed example and is
 * "parity unpinned" beyond those checks.
 */
#ifndef SEER_ORACLE_H
#define SEER_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

double so_bf16_to_f64(uint16_t bits);

/* Threads OpenMP will use in the batched calls (1 when built without OpenMP). */
int so_max_threads(void);

/* D1 for one (b, head): kpool[j][c] = (1/bs) sum_{t in block j} K[t][c] for j < L / bs. */
int so_pool_k(const uint16_t *k, int64_t row_stride, int L, int d, int bs, double *kpool);

/* D2 + D3 for one KV head: q holds the G query rows of its group. */
int so_gate_scores(const uint16_t *q, int64_t q_row_stride, int G, int d,
                   const uint16_t *wq, const uint16_t *wk, int dg,
                   const double *kpool, int nc, double gate_scale,
                   double *s_head /* nullable, [G][nc] */, double *S /* [nc] */);

/* D4: returns the number selected (min(k, nc)); idx ascending. */
int so_select_blocks(const double *S, int nc, int k, int32_t *idx);

/* S1, selection policies beyond the token budget (SeerAttention v2 abstract:
 * the gate adapts to varying sparsity ratios).  The count kept, then the same
 * rule as D4 (largest scores, ties toward the lower id, ids ascending):
 *   policy 0 (budget)     k = min(k_max, nc)
 *   policy 1 (ratio)      k = min(k_max, ceil(nc * num / den))
 *   policy 2 (threshold)  k = min(k_max, #{j < nc : p_j >= tau}),
 *                         p_j = exp(S_j - max S) / sum_i exp(S_i - max S)
 * Returns k, or a negative value on bad arguments. */
int so_select_policy(const double *S, int nc, int policy, int k_max, int num, int den, double tau, int32_t *idx);

/* D5 + D6 for one KV head.  idx: ascending distinct complete-block ids.
 * w (nullable) receives the softmax weight of every token 0..L-1 (0 outside T).
 * An empty T gives out = 0 and lse = -inf. */
int so_sparse_attention(const uint16_t *q, int64_t q_row_stride, int G, int d,
                        const uint16_t *k, const uint16_t *v, int64_t kv_row_stride,
                        int L, int bs, const int32_t *idx, int n_idx, double scale,
                        double *out /* [G][d] */, double *lse /* [G] */,
                        double *w /* nullable, [G][L] */);

/* G1, the block-level ground truth of decoding attention (SeerAttention v2
 * abstract: the block-level ground truth of the attention map, extracted next
 * to the attention itself).  Dense softmax attention of the group's G query
 * rows over the whole context [0, L) (every complete block plus the tail);
 * mass[j] = (1/G) sum_h sum_{t in block j} w_ht for j < nc = L / bs, and
 * mass[nc] = the same sum over the tail [nc*bs, L) (0 when there is none).
 * out [G][d] and lse [G] are that dense attention's.  mass has nc + 1 slots. */
int so_decode_block_mass(const uint16_t *q, int64_t q_row_stride, int G, int d,
                         const uint16_t *k, const uint16_t *v, int64_t kv_row_stride,
                         int L, int bs, double scale, double *out, double *lse, double *mass);

/* D1 over a batch: kpool [B][Hkv][nb_max][d], complete blocks filled, the rest zero. */
int so_pool_cache(const uint16_t *k, int64_t sk_b, int64_t sk_h, int64_t sk_t,
                  const int32_t *seqlens, int B, int Hkv, int d, int bs, int nb_max,
                  double *kpool);

/* D2..D6 over a batch, OpenMP over (b, kvh).  Query head h belongs to KV head h / G.
 * scores [B][Hkv][nb_max] (nullable; -inf past nc), idx [B][Hkv][budget/bs] padded with -1,
 * n_sel [B][Hkv], out [B][Hq][d], lse [B][Hq]. */
int so_decode_step(const uint16_t *q, int64_t sq_b, int64_t sq_h,
                   const uint16_t *k, const uint16_t *v, int64_t skv_b, int64_t skv_h, int64_t skv_t,
                   const int32_t *seqlens, int B, int Hq, int Hkv, int d, int bs, int budget,
                   const uint16_t *wq, const uint16_t *wk, int dg, double gate_scale,
                   const double *kpool, int nb_max, double softmax_scale,
                   double *scores, int32_t *idx, int32_t *n_sel, double *out, double *lse);

/* V1, per-query-head selection (the alternative to D3's shared group
 * selection): every query head keeps its own k = min(budget / bs, nc) blocks
 * by its own gate score s_hj (D2, no group mean) and attends only those (plus
 * the tail).  scores [B][Hq][nb_max] (nullable; -inf past nc), idx
 * [B][Hq][budget/bs] padded with -1, n_sel [B][Hq], out [B][Hq][d], lse [B][Hq]. */
int so_decode_step_per_head(const uint16_t *q, int64_t sq_b, int64_t sq_h,
                            const uint16_t *k, const uint16_t *v, int64_t skv_b, int64_t skv_h, int64_t skv_t,
                            const int32_t *seqlens, int B, int Hq, int Hkv, int d, int bs, int budget,
                            const uint16_t *wq, const uint16_t *wk, int dg, double gate_scale,
                            const double *kpool, int nb_max, double softmax_scale,
                            double *scores, int32_t *idx, int32_t *n_sel, double *out, double *lse);

/* P1..P3 for one head.  nb = ceil(L / bs); S (nullable) [nb][nb], -inf above the diagonal.
 * kv_blocks [nb][kmax_row] ascending, padded with -1; kv_count [nb]. */
int so_prefill_gate(const uint16_t *q, const uint16_t *k, int64_t row_stride, int L, int d, int bs,
                    const uint16_t *wq, const uint16_t *wk, int dg, double gate_scale,
                    int keep_num, int keep_den, double *S, int32_t *kv_blocks, int32_t *kv_count,
                    int kmax_row);

/* P4 for one head, query tokens [t_lo, t_hi): out [t_hi - t_lo][d], lse [t_hi - t_lo]. */
int so_prefill_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t row_stride,
                         int L, int d, int bs, const int32_t *kv_blocks, const int32_t *kv_count,
                         int kmax_row, double scale, int t_lo, int t_hi, double *out, double *lse);

/* P1..P4 over [B][H] heads, OpenMP over heads; query tokens [t_lo, t_hi) of every head.
 * q/k/v [B][H][L][d] contiguous; kv_blocks [B][H][nb][kmax_row]; out [B][H][t_hi-t_lo][d]. */
int so_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v, int B, int H, int L, int d,
               int bs, const uint16_t *wq, const uint16_t *wk, int dg, double gate_scale,
               int keep_num, int keep_den, int32_t *kv_blocks, int32_t *kv_count, int kmax_row,
               double scale, int t_lo, int t_hi, double *out, double *lse);

/* G2, the block-level ground truth of prefill attention (same source as G1):
 * dense causal softmax attention of one head, and for query blocks i in
 * [i_lo, i_hi) and key blocks j <= i the mean over block i's rows t of the
 * weight row t gives to the tokens of block j (t' <= t).  nb = ceil(L / bs);
 * mass [(i_hi - i_lo)][nb], zero for j > i; each row block sums to 1. */
int so_prefill_block_mass(const uint16_t *q, const uint16_t *k, int64_t row_stride, int L, int d, int bs,
                          double scale, int i_lo, int i_hi, double *mass);

#ifdef __cplusplus
}
#endif
#endif
