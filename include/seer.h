/*
 * seer.h -- C ABI of the gfx950 (MI355X) gated block-sparse attention library.
 *
 * The method: "SeerAttention-R: Sparse Attention Adaptation for Long
 * Reasoning" (abstract) decodes with a learned gate that scores every KV block
 * from the current, un-pooled query and the block's pooled key, keeps the
 * best blocks up to a token budget (64- or 128-token blocks), and runs a
 * sparse decoding kernel over the kept blocks only.  Its parent,
 * "SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs"
 * (abstract v1), pools Q and K along the sequence, projects both through
 * learnable linear layers and multiplies them into block scores that drive a
 * block-sparse attention kernel for prefill.
 *
 * Conventions shared by every call
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or keeps device memory; scratch space is passed
 *    in as a caller-owned workspace whose minimum size a *_workspace_size
 *    call reports.
 *  - bf16 tensors are raw bit patterns (seer_bf16).  Strides are in elements;
 *    the innermost (head_dim) dimension is always contiguous.  bf16 base
 *    pointers and row strides must give 16-byte aligned rows.
 *  - Every call validates its host-side arguments first and returns a
 *    negative SEER_ERR_* status without launching anything when they are
 *    invalid.  Otherwise it enqueues its kernels on `stream` and returns
 *    SEER_OK without synchronising; a launch failure returns SEER_ERR_LAUNCH.
 *    Device-resident values (context lengths, block ids, counts) cannot be
 *    checked on the host: the kernels clamp them into range so that a bad
 *    value yields wrong numbers, never an out-of-bounds access.
 *  - Calls are thread-safe and keep no state between calls other than a
 *    per-device cache of the compute-unit count.
 *  - Head grouping (GQA): query head h reads KV head h / (Hq / Hkv).
 */
#ifndef SEER_H
#define SEER_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t seer_bf16; /* raw bfloat16 bits */

enum {
    SEER_OK = 0,
    SEER_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment, bad stride */
    SEER_ERR_UNSUPPORTED = -2, /* valid but not compiled for (head_dim, block size, group) */
    SEER_ERR_WORKSPACE = -3,   /* workspace pointer null or smaller than required */
    SEER_ERR_LAUNCH = -4       /* a kernel launch failed (hipGetLastError) */
};

enum { SEER_OUT_BF16 = 0, SEER_OUT_F32 = 1 };

/* Element type of the pooled-key table. */
enum { SEER_KPOOL_F32 = 0, SEER_KPOOL_BF16 = 1 };

/*
 * How many blocks a (b, head) keeps ("SeerAttention: Learning Intrinsic Sparse
 * Attention in Your LLMs", abstract v2: the gate adapts to varying sparsity
 * ratios; "SeerAttention-R", abstract: a token budget).  With nc complete
 * blocks and the row width k_max of block_idx:
 *   SEER_SELECT_BUDGET     k = min(k_max, nc)          (k_max = budget / block size)
 *   SEER_SELECT_RATIO      k = min(k_max, nc, ceil(nc * ratio_num / ratio_den))
 *   SEER_SELECT_THRESHOLD  k = min(k_max, #{j < nc : p_j >= threshold}),
 *                          p_j = exp(S_j - max S) / sum_i exp(S_i - max S) in fp32
 * then, as always, the k largest scores, ties toward the lower block id, ids
 * ascending.  A NULL policy means the budget.  ratio_den > 0, ratio_num >= 0,
 * threshold not NaN.
 */
enum { SEER_SELECT_BUDGET = 0, SEER_SELECT_RATIO = 1, SEER_SELECT_THRESHOLD = 2 };
typedef struct {
    int kind;
    int ratio_num, ratio_den;
    float threshold;
} seer_select_policy;

/* Human-readable name of a status code (static storage). */
const char *seer_status_string(int status);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
int seer_version(void);

/*
 * Pooled-key cache update (the gate's K pooling: SeerAttention v1 abstract
 * pools K along the sequence, one vector per block; the pooling is the mean).
 *
 *   kpool[b][h][j][:] = (1 / block_size) * sum_{t = j*bs}^{j*bs + bs - 1} K[b][h][t][:]
 *
 * for every listed (b = upd_b[i], j = upd_blk[i]) and every KV head h.
 *   k          bf16 [B][Hkv][kv_capacity][d] with strides sk_b, sk_h, sk_t
 *   upd_b, upd_blk  int32 [n_upd], device; entries out of range are skipped
 *   kpool      fp32 [B][Hkv][nb_max][d], dense; only listed rows are written
 * d in {64, 128}; block_size in {64, 128}.  n_upd == 0 is a no-op.
 * Results are bitwise deterministic, so updating blocks one at a time equals
 * pooling them all at once.
 */
int seer_pool_k_blocks(const seer_bf16 *k, int64_t sk_b, int64_t sk_h, int64_t sk_t,
                       int B, int Hkv, int d, int block_size, int kv_capacity,
                       const int32_t *upd_b, const int32_t *upd_blk, int n_upd,
                       float *kpool, int nb_max, hipStream_t stream);
/* The same into an fp32 (SEER_KPOOL_F32) or bf16 (SEER_KPOOL_BF16: the fp32
 * mean rounded to nearest even; half the gate's bytes) table [B][Hkv][nb_max][d]. */
int seer_pool_k_blocks_ex(const seer_bf16 *k, int64_t sk_b, int64_t sk_h, int64_t sk_t,
                          int B, int Hkv, int d, int block_size, int kv_capacity,
                          const int32_t *upd_b, const int32_t *upd_blk, int n_upd,
                          void *kpool, int kpool_dtype, int nb_max, hipStream_t stream);

/*
 * Gate scores of one decode step (SeerAttention-R abstract: the gate keeps
 * K pooling but drops query pooling, so it reads the current query as is).
 * For sequence b and KV head g with query heads h in g's group:
 *
 *   scores[b][g][j] = mean_h (Wq[g] q[b][h]) . (Wk[g] kpool[b][g][j]) * gate_scale   for j < nc_b
 *   scores[b][g][j] = -inf                                                            for nc_b <= j < nb_max
 *
 * with nc_b = seqlens[b] / block_size complete blocks.  The kernel evaluates
 * the algebraically equal form (Wk[g]^T Wq[g] qbar) . kpool_j, qbar the group
 * mean query, in fp32, in a single launch.
 *   q        bf16 [B][Hq][d] with strides sq_b, sq_h
 *   wq, wk   bf16 [Hkv][dg][d], dense (the gate's linear layers)
 *   kpool    fp32 [B][Hkv][nb_max][d], dense (from seer_pool_k_blocks)
 *   seqlens  int32 [B], device; context length including the current token
 *   scores   fp32 [B][Hkv][nb_max], dense
 * d in {64, 128}; 1 <= dg <= 256; Hq % Hkv == 0; B * Hkv <= 65535.
 */
int seer_gate_scores(const seer_bf16 *q, int64_t sq_b, int64_t sq_h,
                     const seer_bf16 *wq, const seer_bf16 *wk, int dg,
                     const float *kpool, int nb_max, const int32_t *seqlens,
                     int B, int Hq, int Hkv, int d, int block_size, float gate_scale,
                     float *scores, hipStream_t stream);

/*
 * Token-budget block selection (SeerAttention-R abstract: a fixed token
 * budget at 64/128-token block granularity).  Per (b, head):
 *   k = min(budget_tokens / block_size, nc_b); keep the k blocks j < nc_b with
 *   the largest scores, equal scores ordered by the lower block id; write them
 *   ascending to block_idx[b][h][0..k) and -1 to the rest of the row.
 *   scores     fp32 [B][H][nb_max] (finite for j < nc_b)
 *   block_idx  int32 [B][H][budget_tokens / block_size]  (may be NULL when that is 0)
 *   n_sel      int32 [B][H]
 * nb_max <= 16128.
 */
int seer_select_blocks(const float *scores, const int32_t *seqlens, int B, int H, int nb_max,
                       int block_size, int budget_tokens, int32_t *block_idx, int32_t *n_sel,
                       hipStream_t stream);
/* The same with a selection policy; k_max is the row width of block_idx. */
int seer_select_blocks_ex(const float *scores, const int32_t *seqlens, int B, int H, int nb_max,
                          int block_size, int k_max, const seer_select_policy *policy,
                          int32_t *block_idx, int32_t *n_sel, hipStream_t stream);

/*
 * Gate scores and token-budget selection together: the results of
 * seer_gate_scores followed by seer_select_blocks on the scores it wrote
 * (H = Hkv), arguments as there.  When B * Hkv is at least a quarter of the
 * device's compute units, Hq / Hkv is 1, 2, 4 or 8 and nb_max <= 12288, one workgroup per
 * (b, KV head) computes the scores and selects from them in LDS in a single
 * launch; otherwise the two calls run.  The one-launch form reduces u in
 * another order, so its scores may differ from seer_gate_scores' in the last
 * bits; its selection is always exactly seer_select_blocks' on the scores it
 * returns.
 */
int seer_gate_select(const seer_bf16 *q, int64_t sq_b, int64_t sq_h,
                     const seer_bf16 *wq, const seer_bf16 *wk, int dg,
                     const float *kpool, int nb_max, const int32_t *seqlens,
                     int B, int Hq, int Hkv, int d, int block_size, float gate_scale, int budget_tokens,
                     float *scores, int32_t *block_idx, int32_t *n_sel, hipStream_t stream);
/* The same with a selection policy (k_max: row width of block_idx) and the
 * pooled-key table's element type (SEER_KPOOL_BF16: see seer_pool_k_blocks_ex;
 * always one launch, nb_max <= 12288). */
int seer_gate_select_ex(const seer_bf16 *q, int64_t sq_b, int64_t sq_h,
                        const seer_bf16 *wq, const seer_bf16 *wk, int dg,
                        const void *kpool, int kpool_dtype, int nb_max, const int32_t *seqlens,
                        int B, int Hq, int Hkv, int d, int block_size, float gate_scale,
                        int k_max, const seer_select_policy *policy,
                        float *scores, int32_t *block_idx, int32_t *n_sel, hipStream_t stream);

/*
 * Sparse decode over the kept blocks (SeerAttention-R abstract: the sparse
 * decoding kernel reads only the gate's blocks).  For query head h of
 * sequence b, with KV head g = h / G, the token set is
 *   T = union over i < n_sel[b][g] of [block_idx[b][g][i] * bs, + bs)  plus the tail [nc_b * bs, seqlens[b])
 * and the result is softmax attention over T:
 *   out[b][h] = sum_{t in T} softmax_t(softmax_scale * q[b][h] . K[b][g][t]) V[b][g][t]
 *   lse[b][h] = log sum_{t in T} exp(softmax_scale * q[b][h] . K[b][g][t])
 * An empty T gives out = 0 and lse = -inf.  The kept blocks of each (b, g)
 * are split over `num_splits` workgroups (at most 128) whose partial results a
 * second kernel merges by log-sum-exp (num_splits = 0 picks a count from the
 * shape and the device).
 *   q          bf16 [B][Hq][d] with strides sq_b, sq_h
 *   k, v       bf16 [B][Hkv][kv_capacity][d], both with strides skv_b, skv_h, skv_t
 *   seqlens    int32 [B]; block_idx int32 [B][Hkv][k_max]; n_sel int32 [B][Hkv]
 *   out        [B][Hq][d] dense, bf16 (SEER_OUT_BF16) or fp32 (SEER_OUT_F32)
 *   lse        fp32 [B][Hq] or NULL
 *   workspace  >= seer_sparse_decode_workspace_size(...) bytes of fp32 partial
 *              results (none is needed, size 0, when a single split is used)
 * d in {64, 128}; block_size in {64, 128}; Hq / Hkv in {1, 2, 4, 8};
 * softmax_scale > 0 and finite (else SEER_ERR_INVALID_ARG).
 * Only cache rows t < seqlens[b] are read: rows between the context end and
 * kv_capacity (which need not be a multiple of block_size) may hold anything,
 * NaN included.  The K/V rows of one (b, KV head) are addressed with 32-bit
 * byte offsets: kv_capacity * skv_t * 2 must stay below 2^31, else
 * SEER_ERR_UNSUPPORTED (the same limit holds for every call below that reads
 * the K/V cache).
 */
int seer_sparse_decode_num_splits(int B, int Hkv, int k_max, int block_size, int num_splits);
size_t seer_sparse_decode_workspace_size(int B, int Hq, int Hkv, int d, int k_max, int block_size,
                                         int num_splits);
int seer_sparse_decode(const seer_bf16 *q, int64_t sq_b, int64_t sq_h,
                       const seer_bf16 *k, const seer_bf16 *v, int64_t skv_b, int64_t skv_h, int64_t skv_t,
                       int kv_capacity, const int32_t *seqlens, const int32_t *block_idx,
                       const int32_t *n_sel, int k_max, int B, int Hq, int Hkv, int d, int block_size,
                       float softmax_scale, int num_splits, void *workspace, size_t workspace_bytes,
                       void *out, int out_dtype, float *lse, hipStream_t stream);

/*
 * seer_sparse_decode without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and checks as
 * seer_sparse_decode (bit for bit), except that the split partials go to a
 * static device array of SEER_NOALLOC_SCRATCH_BYTES inside the library: each
 * GPU the library runs on holds one such array from the first call on it
 * until the process ends.  The call allocates nothing.  A shape whose
 * partials need more than the array (seer_sparse_decode_workspace_size with
 * the same arguments) returns SEER_ERR_WORKSPACE; a failed lookup of the
 * array's device address returns SEER_ERR_LAUNCH.  Every call on a GPU shares
 * that GPU's array: calls that may overlap on one GPU (on different streams,
 * or from several threads without ordering) race and give wrong results; order
 * them on one stream.
 */
#define SEER_NOALLOC_SCRATCH_BYTES (8u << 20)
int seer_sparse_decode_noalloc(const seer_bf16 *q, int64_t sq_b, int64_t sq_h,
                               const seer_bf16 *k, const seer_bf16 *v, int64_t skv_b, int64_t skv_h, int64_t skv_t,
                               int kv_capacity, const int32_t *seqlens, const int32_t *block_idx,
                               const int32_t *n_sel, int k_max, int B, int Hq, int Hkv, int d, int block_size,
                               float softmax_scale, int num_splits, void *out, int out_dtype, float *lse,
                               hipStream_t stream);

/*
 * Per-query-head selection (the alternative GQA reading): every query head h
 * keeps its own k = min(budget / bs, nc_b) blocks by its own gate score
 * s_hj = gate_scale * (Wq[g] q_h) . (Wk[g] kp_j) (no group mean) and attends
 * only those blocks plus the tail.
 *   seer_gate_select_heads: scores fp32 [B][Hq][nb_max] (-inf past nc_b),
 *     block_idx int32 [B][Hq][budget / bs] ascending, -1 padded, n_sel [B][Hq];
 *     other arguments as seer_gate_select.  Hq / Hkv in {1, 2, 4, 8},
 *     (Hq / Hkv) * nb_max <= 10240.
 *   seer_sparse_decode_heads: out / lse as seer_sparse_decode for these per-head
 *     sets; each block of the union of a group's sets is read once for all of
 *     the group's heads, a head giving no weight to blocks it did not keep.
 *     block_idx / n_sel as written above (k_max = row width), nb_max the
 *     pooled-table width (<= 4096, bounds the block ids); workspace >=
 *     seer_sparse_decode_heads_workspace_size(...) bytes of split partials.
 */
int seer_gate_select_heads(const seer_bf16 *q, int64_t sq_b, int64_t sq_h,
                           const seer_bf16 *wq, const seer_bf16 *wk, int dg,
                           const float *kpool, int nb_max, const int32_t *seqlens,
                           int B, int Hq, int Hkv, int d, int block_size, float gate_scale, int budget_tokens,
                           float *scores, int32_t *block_idx, int32_t *n_sel, hipStream_t stream);
size_t seer_sparse_decode_heads_workspace_size(int B, int Hq, int Hkv, int d, int k_max, int nb_max,
                                               int block_size, int num_splits);
int seer_sparse_decode_heads(const seer_bf16 *q, int64_t sq_b, int64_t sq_h,
                             const seer_bf16 *k, const seer_bf16 *v, int64_t skv_b, int64_t skv_h, int64_t skv_t,
                             int kv_capacity, const int32_t *seqlens, const int32_t *block_idx,
                             const int32_t *n_sel, int k_max, int nb_max,
                             int B, int Hq, int Hkv, int d, int block_size, float softmax_scale, int num_splits,
                             void *workspace, size_t workspace_bytes, void *out, int out_dtype, float *lse,
                             hipStream_t stream);

/*
 * Block-level ground truth of decoding attention ("SeerAttention: Learning
 * Intrinsic Sparse Attention in Your LLMs", abstract v2: the block-level
 * ground truth of the attention map, extracted next to the attention itself;
 * the gate is distilled toward it).  Dense attention of every query head over
 * its whole context [0, seqlens[b]) -- out and lse as seer_sparse_decode with
 * every complete block kept -- and per (b, g) the attention mass of each block,
 * averaged over g's query heads:
 *   mass[b][g][j]      = (1/G) sum_h sum_{t in block j} softmax_t      j < nc_b
 *   mass[b][g][nb_max] = the same sum over the tail [nc_b*bs, seqlens[b])
 *   mass[b][g][j]      = 0 for nc_b <= j < nb_max (and the tail slot without a tail)
 * Each row sums to 1 (0 for an empty context).  nb_max >= seqlens[b] / block_size
 * (blocks past nb_max are not attended).
 *   mass       fp32 [B][Hkv][nb_max + 1]
 *   lse        fp32 [B][Hq] or NULL
 *   workspace  >= seer_decode_block_mass_workspace_size(...) bytes (split
 *              partials, the lse when lse is NULL, and per-block sums)
 * Other arguments and limits as seer_sparse_decode.
 */
size_t seer_decode_block_mass_workspace_size(int B, int Hq, int Hkv, int d, int nb_max, int block_size,
                                             int num_splits);
int seer_decode_block_mass(const seer_bf16 *q, int64_t sq_b, int64_t sq_h,
                           const seer_bf16 *k, const seer_bf16 *v, int64_t skv_b, int64_t skv_h, int64_t skv_t,
                           int kv_capacity, const int32_t *seqlens, int B, int Hq, int Hkv, int d,
                           int block_size, float softmax_scale, int nb_max, int num_splits,
                           void *workspace, size_t workspace_bytes, void *out, int out_dtype, float *lse,
                           float *mass, hipStream_t stream);

/*
 * One whole decode step: the gate scores, the token-budget selection and the
 * sparse decode with its merge, in three kernel launches instead of four: the
 * gate scores; one kernel whose workgroups select their (b, KV head)'s blocks
 * in LDS and decode their split; the merge of the splits (none with a single
 * split).  The results equal those of seer_gate_scores + seer_select_blocks +
 * seer_sparse_decode with the same arguments bit for bit.
 *   arguments as in the three calls above; scores [B][Hkv][nb_max],
 *   block_idx [B][Hkv][budget_tokens / block_size] and n_sel [B][Hkv] are
 *   written as those calls write them.
 *   workspace >= seer_decode_step_workspace_size(...) bytes (the split
 *              partials, as seer_sparse_decode's; may be null when that is 0).
 *              Calls sharing a workspace must be ordered on one stream.
 * nb_max <= 16128; B * Hkv <= 65535.
 */
size_t seer_decode_step_workspace_size(int B, int Hq, int Hkv, int d, int k_max, int block_size,
                                       int num_splits);

/*
 * The second and third launches of seer_decode_step on their own: from given
 * gate scores, the token-budget selection (in the decode kernel's LDS) and the
 * sparse decode, then the merge of the splits.  Results equal
 * seer_select_blocks + seer_sparse_decode with the same arguments bit for bit.
 *   scores [B][Hkv][nb_max] fp32 (as seer_gate_scores writes them; entries past
 *   a sequence's complete blocks are not read); the other arguments as in
 *   seer_decode_step, workspace as seer_sparse_decode_workspace_size reports.
 */
int seer_select_sparse_decode(const seer_bf16 *q, int64_t sq_b, int64_t sq_h,
                              const seer_bf16 *k, const seer_bf16 *v, int64_t skv_b, int64_t skv_h, int64_t skv_t,
                              int kv_capacity, const int32_t *seqlens, const float *scores, int nb_max,
                              int B, int Hq, int Hkv, int d, int block_size, int budget_tokens,
                              float softmax_scale, int num_splits, int32_t *block_idx, int32_t *n_sel,
                              void *workspace, size_t workspace_bytes, void *out, int out_dtype, float *lse,
                              hipStream_t stream);
int seer_decode_step(const seer_bf16 *q, int64_t sq_b, int64_t sq_h,
                     const seer_bf16 *k, const seer_bf16 *v, int64_t skv_b, int64_t skv_h, int64_t skv_t,
                     int kv_capacity, const int32_t *seqlens,
                     const seer_bf16 *wq, const seer_bf16 *wk, int dg, float gate_scale,
                     const float *kpool, int nb_max, int B, int Hq, int Hkv, int d, int block_size,
                     int budget_tokens, float softmax_scale, int num_splits,
                     float *scores, int32_t *block_idx, int32_t *n_sel,
                     void *workspace, size_t workspace_bytes, void *out, int out_dtype, float *lse,
                     hipStream_t stream);

/*
 * Block-sparse causal prefill (SeerAttention, abstract v1: the gate pools Q and
 * K per block, projects both through learnable linear layers and multiplies
 * them into block scores; a block-sparse FlashAttention kernel attends only
 * the activated blocks).  Per (b, h), with nb = ceil(L / block_size) blocks:
 *
 *   Qbar_i, Kbar_j   mean of the rows of block i / j (a partial last block:
 *                    mean of the rows it has)
 *   S_ij = gate_scale * (Wq[h] Qbar_i) . (Wk[h] Kbar_j)          j <= i
 *   row i keeps k_i = ceil((i + 1) * keep_num / keep_den) blocks (at least 1,
 *   at most i + 1): the diagonal block i plus the k_i - 1 best j < i, equal
 *   scores ordered by the lower id; kv_blocks[b][h][i][0..k_i) lists them in
 *   ascending order (so the diagonal last), -1 after; kv_count[b][h][i] = k_i.
 *   out[b][h][t] = softmax attention of query token t (in block i) over the
 *   tokens t' <= t of row i's kept blocks, scale softmax_scale;
 *   lse[b][h][t] = log of its softmax denominator (natural log).
 *
 * With use_given_blocks != 0 the gate is skipped: kv_blocks / kv_count are
 * inputs (ids are clamped into [0, i]; counts into [0, kmax_row]; a row with
 * count 0 gives zeros and lse = -inf) and wq, wk, workspace may be NULL.
 *   q, k, v, out  bf16 [B][H][L][d], dense
 *   wq, wk        bf16 [H][dg][d], dense
 *   kv_blocks     int32 [B][H][nb][kmax_row]; kv_count int32 [B][H][nb]
 *   lse           fp32 [B][H][L] or NULL
 *   workspace     >= seer_block_sparse_prefill_workspace_size(...) bytes: fp32
 *                 projected pooled Q and K (rows padded to 128 or 256 floats)
 *                 and, beyond 2048 blocks only, the block score matrix
 * d = 128, block_size = 64, 1 <= dg <= 256; without given blocks,
 * kmax_row >= seer_block_sparse_prefill_kmax_row(L, block_size, keep_num, keep_den)
 * and nb <= 16128.
 */
int seer_block_sparse_prefill_kmax_row(int L, int block_size, int keep_num, int keep_den);
size_t seer_block_sparse_prefill_workspace_size(int B, int H, int L, int d, int block_size, int dg);
int seer_block_sparse_prefill(const seer_bf16 *q, const seer_bf16 *k, const seer_bf16 *v,
                              int B, int H, int L, int d, int block_size,
                              const seer_bf16 *wq, const seer_bf16 *wk, int dg, float gate_scale,
                              int keep_num, int keep_den, int32_t *kv_blocks, int32_t *kv_count,
                              int kmax_row, int use_given_blocks, float softmax_scale,
                              void *workspace, size_t workspace_bytes, seer_bf16 *out, float *lse,
                              hipStream_t stream);

/*
 * Block-level ground truth of prefill attention ("SeerAttention: Learning
 * Intrinsic Sparse Attention in Your LLMs", abstract v2: the block-level
 * ground truth of the attention map, extracted next to the attention with a
 * customised FlashAttention).  Dense causal attention (out, lse as
 * seer_block_sparse_prefill with every causal block kept), then for query
 * block i and key block j <= i
 *   mass[b][h][i][j] = mean over the rows t of block i of sum_{t' in block j, t' <= t} softmax_t(t')
 * and 0 for j > i; each row block sums to 1.
 *   mass  fp32 [B][H][nb][nb], nb = ceil(L / block_size); lse may be NULL
 * d = 128, block_size = 64.
 */
int seer_prefill_block_mass(const seer_bf16 *q, const seer_bf16 *k, const seer_bf16 *v, int B, int H, int L,
                            int d, int block_size, float softmax_scale, seer_bf16 *out, float *lse, float *mass,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SEER_H */
