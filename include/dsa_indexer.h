/*
 * dsa_indexer.h -- C ABI of the DeepSeek Sparse Attention (DSA) indexer hot path on MI355X
 * (gfx950): store compressed index keys into a paged cache, score queries against every causally
 * visible key, select the top-k keys per query.
 *
 * The operation is the indexer the four DSA-indexer blog pages describe:
 *  - "When the Fused Kernel Isn't Enough", Input Knowledge Required: a store path writes compressed
 *    keys, a read path loads them and computes logits; an fp8 key is 128 B of codes + a 4 B scale
 *    (132 B/token), a bf16 key is 256 B/token.
 *  - "The Moment of Validation", Input Knowledge Required: the fused store normalises, applies RoPE
 *    and writes the cache; fp8 keys share one scale per group (here: per key).
 *  - "The Crash That Changed Direction", Experiment and Assumptions: the scores are a batched q.k
 *    product followed by ReLU over the head dimension, then top-k; fp8 keys are e4m3 and widen
 *    exactly to bf16 before the product.
 *  - "The Fused Kernel Decision", Message and Assumptions: the cache is paged, 64 keys per page,
 *    [npages, 64*128]; a key maps to (page, offset); q and k share one element order.
 *  - "When the Fused Kernel Isn't Enough", Message and Why This Message Matters: materialising the
 *    full per-head logits tensor is what ran out of memory at 22K tokens; this library never does.
 *
 * Conventions for every entry point:
 *  - Pointers named "device" are device (HBM) memory the caller owns; the library never allocates
 *    or frees device memory and keeps no state between calls.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream) without a host
 *    synchronisation.  The return value reports host-side argument validation and launch errors;
 *    a fault inside a kernel surfaces at the caller's next synchronisation.
 *  - Integers inside device arrays are read as given; out-of-range values never cause an
 *    out-of-bounds access (see each entry point for what they do instead).
 *  - head_dim is 128, n_heads is 64, 64 keys per page, 4 tokens per compressed key.
 */
#ifndef DSA_INDEXER_H
#define DSA_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IDX_ABI_VERSION 1
#define IDX_HEAD_DIM 128
#define IDX_N_HEADS 64
#define IDX_PAGE_KEYS 64
#define IDX_COMPRESS_RATIO 4
#define IDX_MAX_TOPK 2048

typedef enum {
  IDX_OK = 0,
  IDX_EINVAL = 1,        /* a null pointer, negative size or out-of-range scalar argument */
  IDX_EUNSUPPORTED = 2,  /* a valid but unsupported configuration (n_heads != 64, dtype) */
  IDX_EWORKSPACE = 3,    /* the workspace is smaller than one query row needs */
  IDX_EHIP = 4           /* a HIP launch returned an error */
} idx_status;

typedef enum {
  IDX_KV_FP8_E4M3 = 0,   /* page = 64 x 128 e4m3fn codes, then 64 fp32 scales: 8448 B */
  IDX_KV_BF16 = 1,       /* page = 64 x 128 bf16: 16384 B */
  IDX_KV_FP4_E2M1 = 2    /* page = 64 x 64 bytes of e2m1 code pairs, then 64 fp32 scales: 4352 B */
} idx_kv_dtype;

/* IDX_ABI_VERSION of the built library. */
int idx_abi_version(void);

/* Static text for a status code (never NULL). */
const char* idx_status_string(int status);

/* Bytes of one cache page for `dtype` (8448 for fp8, 16384 for bf16, 4352 for fp4), 0 for an
 * unknown dtype.  Per key: 128 code bytes + a 4 B fp32 scale, or 256 bf16 bytes ("When the Fused
 * Kernel Isn't Enough", Input Knowledge Required).  Inside an fp8 page the 64 code rows come
 * first (16 B aligned for vector loads), then the 64 scales.  fp4 ("The Fused Kernel Decision",
 * Input Knowledge: an fp4 variant of the indexer for more compression; the format is this
 * library's choice): OCP e2m1 codes (sign, 2 exponent bits with bias 1, 1 mantissa bit; largest
 * 6), dims 2i and 2i+1 in the low and high nibble of byte i, 64 B per key, then the 64 fp32
 * scales; 68 B per key. */
size_t idx_page_bytes(int dtype);

/*
 * S1 -- fused RMSNorm + RoPE + quantise + paged store of compressed index keys ("The Moment of
 * Validation", Input Knowledge Required; "The Fused Kernel Decision", Message).
 *
 * For each input row n (key s = key_idx[n] of sequence b = key_seq[n]):
 *   y   = x[n] / sqrt(mean(x[n]^2) + eps) * gamma           (fp64 inside the kernel)
 *   rotate dims (64+2j, 65+2j), j = 0..31, by angle 4*s * inv_freq_j,
 *       inv_freq_j = fp32(10000^(-2j/64))                    (RoPE position = first token, 4s)
 *   k32 = y rounded once to fp32
 *   bf16: code_i = RNE bf16 of k32_i
 *   fp8:  scale = fp32(max_i |k32_i| / 448); code_i = e4m3fn RNE, saturating, of fp32(k32_i/scale);
 *         an all-zero key stores scale 0 and codes 0
 *   fp4:  scale = fp32(max_i |k32_i| / 6); code_i = e2m1 RNE, saturating, of fp32(k32_i/scale);
 *         an all-zero key stores scale 0 and codes 0
 * and writes the key to slot s % 64 of page page_table[b * max_pages + s / 64] of `kcache`.
 *
 * x          device fp32 [n_keys, 128], row-major, 16-byte aligned
 * gamma      device fp32 [128], 16-byte aligned
 * eps        RMSNorm epsilon (added to the mean square)
 * key_idx    device int32 [n_keys]
 * key_seq    device int32 [n_keys], or NULL: every key belongs to sequence 0
 * page_table device int32 [n_seq, max_pages]; -1 = no page
 * kcache     device, n_pages_pool * idx_page_bytes(dtype) bytes; only the addressed slots (and, for
 *            fp8, their scale words) are written
 * Rows whose sequence, key index (>= max_pages * 64) or page id (outside [0, n_pages_pool)) is out
 * of range are skipped.  Two rows that address the same slot race.  n_keys == 0 is a no-op.
 * Errors: IDX_EINVAL (null pointer or misaligned x / gamma / kcache with n_keys > 0,
 * n_keys/n_seq/max_pages/n_pages_pool < 0 or eps < 0), IDX_EUNSUPPORTED (unknown dtype), IDX_EHIP.
 */
int idx_store_keys(const float* x, const float* gamma, float eps, const int32_t* key_idx,
                   const int32_t* key_seq, int64_t n_keys, const int32_t* page_table,
                   int32_t n_seq, int32_t max_pages, int dtype, void* kcache,
                   int64_t n_pages_pool, void* stream);

/*
 * S1, rotated store: as idx_store_keys, with the key multiplied after RoPE (still in fp64, before
 * the rounding to fp32) by the normalised 128-point Walsh-Hadamard matrix H / sqrt(128),
 * H[i][j] = (-1)^popcount(i & j) ("When the Fused Kernel Isn't Enough", the fused vs. non-fused
 * paths: the fused kernel applies normalisation, RoPE and the Hadamard transform before the
 * store; "The Fused Kernel Decision", Assumptions: q and k must go through the same transform and
 * element order).  Scores against such a cache need q rotated by idx_rotate_q; q.k is then the
 * unrotated product up to the roundings.  Arguments and errors as idx_store_keys.
 */
int idx_store_keys_rotated(const float* x, const float* gamma, float eps, const int32_t* key_idx,
                           const int32_t* key_seq, int64_t n_keys, const int32_t* page_table,
                           int32_t n_seq, int32_t max_pages, int dtype, void* kcache,
                           int64_t n_pages_pool, void* stream);

/*
 * q for a rotated cache: each of n_vec 128-dim bf16 vectors (a [n_q, 64, 128] q is n_q * 64
 * vectors) multiplied by H / sqrt(128) in fp64, rounded to fp32 and then to bf16 (nearest-even).
 * q          device bf16 [n_vec, 128], 16-byte aligned
 * out        device bf16 [n_vec, 128], 16-byte aligned; may be q itself (in place)
 * Errors: IDX_EINVAL (null or misaligned pointer with n_vec > 0, n_vec < 0), IDX_EHIP.  n_vec == 0
 * is a no-op.
 */
int idx_rotate_q(const void* q, void* out, int64_t n_vec, void* stream);

/*
 * Bytes of workspace idx_logits_topk uses for a call of this shape when the caller wants all
 * queries scored in one pass.  Any workspace of at least idx_logits_topk_min_workspace() bytes
 * works: the call then processes the queries in chunks that fit.  The bound never depends on
 * n_heads: per-head logits are never materialised.
 */
size_t idx_logits_topk_workspace_size(int64_t n_q, int32_t n_seq, int32_t max_pages, int32_t k);
size_t idx_logits_topk_min_workspace(int32_t n_seq, int32_t max_pages, int32_t k);

/*
 * Host only (no HIP call): the query chunking idx_logits_topk (and idx_logits_topk_fp8q) uses
 * for a workspace of workspace_bytes, so that a caller can see how a budget is spent before
 * launching.  n_seq as for the call (it decides which selection a batch shape gets).
 * rows_per_chunk   out: query rows scored and selected per chunk (the last chunk may be smaller;
 *                  the smaller of the two calls' chunkings)
 * max_chunk_bytes  out: the most workspace bytes any chunk of the call touches; never more than
 *                  workspace_bytes when the status is IDX_OK
 * Errors: IDX_EINVAL (null output, n_q < 1, n_seq < 0, max_pages < 0, k outside
 * [1, IDX_MAX_TOPK]),
 * IDX_EWORKSPACE (not even one query row fits; rows_per_chunk is then 0).
 */
int idx_logits_topk_plan(int64_t n_q, int32_t n_seq, int32_t max_pages, int32_t k,
                         size_t workspace_bytes, int64_t* rows_per_chunk,
                         size_t* max_chunk_bytes);

/*
 * S2 + S3 -- score every query against every causally visible key and select the top-k
 * ("The Crash That Changed Direction", Input Knowledge Required and Pivot; top-k 512 and 1024,
 * "The Crash That Changed Direction", Context).
 *
 * Queries of sequence b are its last q_len_b = cu_q[b+1] - cu_q[b] tokens: row i of q with
 * cu_q[b] <= i < cu_q[b+1] sits at token t = seq_lens[b] - q_len_b + (i - cu_q[b]) and sees keys
 * s < n_vis = min(floor((t+1)/4), max_pages*64) (key s covers tokens 4s..4s+3; t < 0 sees none).
 *   logit(i, s) = sum_h w[i,h] * max(0, sum_d q[i,h,d] * k[s,d])
 * with k the stored key (bf16, or e4m3 code * scale), computed with fp32 accumulation.
 * out_idx[i, :] receives the k keys s with the largest logits (ties to the lower s), in an
 * unspecified order within the row, then -1 padding when n_vis < k; out_val (optional) their
 * logits in the same order, -inf for padding.
 * Keys whose page id lies outside [0, n_pages_pool) score -inf.
 *
 * q          device bf16 [n_q, 64, 128], 16-byte aligned
 * w          device fp32 [n_q, 64]
 * kcache     device pool as written by idx_store_keys with the same dtype (16-byte aligned)
 * page_table device int32 [n_seq, max_pages]
 * seq_lens   device int32 [n_seq]
 * cu_q       device int32 [n_seq + 1], non-decreasing, cu_q[0] = 0, cu_q[n_seq] = n_q
 *            (a row outside every [cu_q[b], cu_q[b+1]) sees no key)
 * out_idx    device int32 [n_q, k];  out_val device fp32 [n_q, k] or NULL
 * workspace  device, 16-byte aligned, workspace_bytes >= idx_logits_topk_min_workspace(...)
 * Errors: IDX_EINVAL (null pointer, misaligned q / kcache / workspace,
 * n_q/n_seq/max_pages/n_pages_pool < 0, k < 1 or k > IDX_MAX_TOPK), IDX_EUNSUPPORTED (n_heads !=
 * 64, unknown dtype), IDX_EWORKSPACE, IDX_EHIP.
 */
int idx_logits_topk(const void* q, const float* w, const void* kcache, int dtype,
                    int64_t n_pages_pool, const int32_t* page_table, int32_t n_seq,
                    int32_t max_pages, const int32_t* seq_lens, const int32_t* cu_q, int64_t n_q,
                    int32_t n_heads, int32_t k, int32_t* out_idx, float* out_val,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * idx_logits_topk for callers that cannot allocate device memory or pass a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  It calls no
 * hipMalloc, hipFree or other allocating routine.  Its workspace is the library's own static
 * device scratch of idx_logits_topk_noalloc_scratch_bytes() bytes (64 MiB), one per GPU, held
 * from the library's load until the process ends; its device address is looked up on the first
 * call on each device (with that device current).  Arguments, results and errors are those of
 * idx_logits_topk; a batch whose full workspace exceeds the scratch is processed in query chunks
 * that fit, and one that cannot fit even one query row returns IDX_EWORKSPACE.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one GPU (different
 * streams, or host threads) race and must be ordered by the caller.  The scratch needs no
 * clearing between calls: every region is written before it is read within a call.
 */
int idx_logits_topk_noalloc(const void* q, const float* w, const void* kcache, int dtype,
                            int64_t n_pages_pool, const int32_t* page_table, int32_t n_seq,
                            int32_t max_pages, const int32_t* seq_lens, const int32_t* cu_q,
                            int64_t n_q, int32_t n_heads, int32_t k, int32_t* out_idx,
                            float* out_val, void* stream);
size_t idx_logits_topk_noalloc_scratch_bytes(void);

/*
 * idx_logits_topk with instrumentation: `ev_score_begin` / `ev_score_end` (hipEvent_t, either may
 * be NULL) are recorded on `stream` right before the first and right after the last launch of the
 * scoring kernel, so a caller can time that kernel alone.  Results are identical.
 */
int idx_logits_topk_timed(const void* q, const float* w, const void* kcache, int dtype,
                          int64_t n_pages_pool, const int32_t* page_table, int32_t n_seq,
                          int32_t max_pages, const int32_t* seq_lens, const int32_t* cu_q,
                          int64_t n_q, int32_t n_heads, int32_t k, int32_t* out_idx,
                          float* out_val, void* workspace, size_t workspace_bytes,
                          void* ev_score_begin, void* ev_score_end, void* stream);

/*
 * S2 alone, for checking: out_logits[i, s] (device fp32 [n_q, max_keys], row stride max_keys)
 * receives logit(i, s) for visible s < max_keys and -inf for every other s < max_keys.  Uses the
 * same scoring kernel as idx_logits_topk, so its values are bit-identical to the ones top-k
 * selects from.  Materialises the head-reduced [n_q, max_keys] matrix; never the per-head one.
 * Arguments and errors as idx_logits_topk; max_keys < 1 is IDX_EINVAL.
 */
int idx_logits_dense(const void* q, const float* w, const void* kcache, int dtype,
                     int64_t n_pages_pool, const int32_t* page_table, int32_t n_seq,
                     int32_t max_pages, const int32_t* seq_lens, const int32_t* cu_q, int64_t n_q,
                     int32_t n_heads, float* out_logits, int32_t max_keys, void* stream);

/*
 * fp8 x fp8 scoring (the fp8 product of "The Crash That Changed Direction", Experiment, taken
 * with q in fp8 as well, on the gfx950 fp8 matrix cores at twice the bf16 rate).
 *
 * idx_quantize_q: each 128-dim bf16 vector of q (one query head; a [n_q, 64, 128] q is n_q * 64
 * vectors) gets one fp32 scale = fp32(max_i |q_i| / 448) and e4m3fn codes = RNE, saturating, of
 * fp32(q_i / scale), the rule of the fp8 key store; an all-zero vector gets scale 0, codes 0.
 * q        device bf16 [n_vec, 128], 16-byte aligned
 * q_codes  device uint8 [n_vec, 128], 16-byte aligned
 * q_scales device fp32 [n_vec]
 * Errors: IDX_EINVAL (null or misaligned pointer with n_vec > 0, n_vec < 0), IDX_EHIP.
 *
 * idx_logits_topk_fp8q / idx_logits_dense_fp8q: as idx_logits_topk / idx_logits_dense against an
 * fp8 cache (IDX_KV_FP8_E4M3; there is no dtype argument), with
 *   logit(i, s) = sum_h w[i,h] * max(0, sum_d (qc[i,h,d] * qs[i,h]) * (kc[s,d] * ks[s]))
 * accumulated in fp32 from the exact products of e4m3 values.  q_codes is uint8 [n_q, 64, 128]
 * (16-byte aligned) and q_scales fp32 [n_q, 64] from idx_quantize_q (or any codes and non-negative scales).  The
 * workspace rules and errors are those of idx_logits_topk; _timed records the two events around
 * the scoring launches like idx_logits_topk_timed.
 */
int idx_quantize_q(const void* q, void* q_codes, float* q_scales, int64_t n_vec, void* stream);
int idx_logits_topk_fp8q(const void* q_codes, const float* q_scales, const float* w,
                         const void* kcache, int64_t n_pages_pool, const int32_t* page_table,
                         int32_t n_seq, int32_t max_pages, const int32_t* seq_lens,
                         const int32_t* cu_q, int64_t n_q, int32_t n_heads, int32_t k,
                         int32_t* out_idx, float* out_val, void* workspace,
                         size_t workspace_bytes, void* stream);
int idx_logits_topk_fp8q_timed(const void* q_codes, const float* q_scales, const float* w,
                               const void* kcache, int64_t n_pages_pool,
                               const int32_t* page_table, int32_t n_seq, int32_t max_pages,
                               const int32_t* seq_lens, const int32_t* cu_q, int64_t n_q,
                               int32_t n_heads, int32_t k, int32_t* out_idx, float* out_val,
                               void* workspace, size_t workspace_bytes, void* ev_score_begin,
                               void* ev_score_end, void* stream);
int idx_logits_dense_fp8q(const void* q_codes, const float* q_scales, const float* w,
                          const void* kcache, int64_t n_pages_pool, const int32_t* page_table,
                          int32_t n_seq, int32_t max_pages, const int32_t* seq_lens,
                          const int32_t* cu_q, int64_t n_q, int32_t n_heads, float* out_logits,
                          int32_t max_keys, void* stream);

/*
 * S3 alone: top-k of each row of a score matrix ("The Crash That Changed Direction", Context and
 * Pivot: the top-k op over indexer logits, k = 512 or 1024).
 *
 * scores   device fp32 [n_rows, row_stride]; row r holds row_len[r] candidates (clamped to
 *          [0, row_stride]; row_len NULL = row_stride each).  Values must not be NaN; -0 and +0
 *          compare equal.
 * out_idx  device int32 [n_rows, k]: the column indices of the k largest values (ties to the lower
 *          index), in an unspecified order within the row, then -1; out_val (optional) device
 *          fp32 [n_rows, k] their values in the same order, then -inf.
 * workspace device, 16-byte aligned, at least idx_topk_rows_workspace_size(n_rows, row_stride, k)
 *          bytes (that size is 0, and workspace may be NULL, when every row is selected in one
 *          pass: batches of at most 128 rows of at most 32768 scores, or rows of at most 6144
 *          scores in batches large enough to fill the GPU).
 * Errors: IDX_EINVAL (null pointer, misaligned workspace, n_rows < 0, row_stride < 1, k < 1 or
 * k > IDX_MAX_TOPK), IDX_EWORKSPACE, IDX_EHIP.
 */
size_t idx_topk_rows_workspace_size(int64_t n_rows, int64_t row_stride, int32_t k);
int idx_topk_rows(const float* scores, int64_t n_rows, int64_t row_stride, const int32_t* row_len,
                  int32_t k, int32_t* out_idx, float* out_val, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * Sparse attention over the selected keys: the consumer of the top-k lists ("When the Fused Kernel
 * Isn't Enough", Input Knowledge: the sparse attention attends to the top-K entries the indexer
 * picks; the main KV cache is bf16 with head_dim 512; "The Fused Kernel Decision", Message: that
 * cache is unpaged, [num_slots, 512] bf16).  The 512-dim latent of an entry is its key and its
 * value for every query head (multi-query attention on the shared latent).  For query row i of
 * sequence b (cu_q[b] <= i < cu_q[b+1]) and head h, the listed entries j < k with
 * 0 <= idx[i,j] < max_keys and slot = kv_slot[b, idx[i,j]] in [0, n_slots) give latents v_j and
 *   logit_j = softmax_scale * sum_d q[i,h,d] * v_j[d]
 *   out[i,h,:] = sum_j softmax_j(logit) * v_j        (bf16, round to nearest even)
 *   out_lse[i,h] = log(sum_j exp(logit_j))           (natural log; optional)
 * A list entry counts once per appearance.  A row with no valid entry gets out = 0 and
 * out_lse = -inf.  Scores accumulate in fp32 from exact bf16 products; the softmax weights are
 * rounded to bf16 for the weighted sum and normalised by the sum of the rounded weights.
 *
 * q        device bf16 [n_q, n_heads, 512], 16-byte aligned
 * kv       device bf16 [n_slots, 512], 16-byte aligned
 * kv_slot  device int32 [n_seq, max_keys]: the kv row of key s of sequence b (out of range: the
 *          entry is skipped)
 * cu_q     device int32 [n_seq + 1], non-decreasing; rows outside [cu_q[0], cu_q[n_seq]) attend
 *          to nothing
 * idx      device int32 [n_q, k], e.g. the output of idx_logits_topk (its -1 padding is skipped)
 * out      device bf16 [n_q, n_heads, 512], 16-byte aligned; out_lse device fp32 [n_q, n_heads]
 *          or NULL
 * workspace device, 16-byte aligned, at least idx_sparse_attn_workspace_size(n_q, n_heads, k)
 *          bytes (0, and workspace may be NULL, when no list is split: batches of 256 rows or
 *          more with k <= 2048, or k <= 1024 with 32 heads)
 * n_heads is 32, 64 or 128.
 * Errors: IDX_EINVAL (null pointer, misaligned q / kv / out / workspace, n_q < 0, n_seq < 1,
 * max_keys < 1, n_slots < 0, k < 1, softmax_scale not finite and positive), IDX_EUNSUPPORTED
 * (n_heads), IDX_EWORKSPACE, IDX_EHIP.
 */
#define IDX_LATENT_DIM 512
size_t idx_sparse_attn_workspace_size(int64_t n_q, int32_t n_heads, int32_t k);
int idx_sparse_attn(const void* q, const void* kv, int64_t n_slots, const int32_t* kv_slot,
                    int32_t n_seq, int32_t max_keys, const int32_t* cu_q, const int32_t* idx,
                    int64_t n_q, int32_t n_heads, int32_t k, float softmax_scale, void* out,
                    float* out_lse, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_INDEXER_H */
