/*
 * dsa.h -- C ABI of libdsa.so, the MI355X (gfx950) DeepSeek Sparse Attention
 * decode path: lightning indexer -> deterministic top-k -> absorbed sparse MLA.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every array argument is a device pointer (HBM), allocated and
 *   owned by the caller; the library never allocates, frees or keeps them.
 *   Scalars are host values. `stream` is a hipStream_t (NULL = the default
 *   stream); every call only enqueues work on it and returns without waiting.
 * Caches.  Indexer keys and latent rows are flat row arrays shared by B
 *   sequences: sequence b owns rows row_off[b] .. row_off[b] + len_b - 1 of
 *   a cache of `cache_rows` rows. Query r belongs to sequence q_seq[r]
 *   (q_seq == NULL means query r belongs to sequence r) at 0-based position
 *   q_pos[r]; its candidate keys are positions 0 .. q_pos[r] of that sequence
 *   (the query's own key included). Decode is R == B, q_seq == NULL,
 *   q_pos[b] = len_b - 1 (or q_per_seq new tokens per sequence, R = B *
 *   q_per_seq, in dsa_decode_fused); causal prefill is B == 1, q_pos[r] = r.
 *   The *_paged entry points take a block table over a pool of fixed-size
 *   pages instead of row_off.
 * Device metadata (row_off, q_seq, q_pos, seq_len, idx) is trusted: the
 *   preconditions q_pos[r] < max_n, 0 <= q_seq[r] < B and
 *   row_off[q_seq[r]] + q_pos[r] < cache_rows are not checked on the host.
 *   Kernels clamp every address so a violation cannot read or write outside
 *   the caller's buffers; the values computed for such queries are then
 *   unspecified.
 * Errors.  Argument errors are found on the host before anything is
 *   enqueued and returned synchronously (nothing is written). A failed
 *   launch returns DSA_ERR_HIP; dsa_last_error() gives its text.
 * Determinism.  For fixed inputs, shapes and device, every output is bitwise
 *   identical from run to run: no floating-point atomics, fixed reduction
 *   orders, and integer-only selection.
 * dtypes.  DSA_BF16 arrays hold bfloat16 bit patterns, DSA_FP8_E4M3 arrays
 *   OCP FP8 E4M3FN codes (max 448, no infinities), DSA_F32 IEEE float32.
 *
 * Citations name the pages that describe the method: "GLM-5: from Vibe
 * Coding to Agentic Engineering" (paper notes, sections 2.1, 2.1.1, 2.1.2,
 * 2.4.2, 3.2), "Zhipu AI / GLM: From Blank Infilling to Compaction-Aware
 * Agentic RL" (sections 9.1, 9.3, 11.1, 11.4) and "GLM-5 Notes" (DSA,
 * Replay).
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,        /* a required pointer is NULL                      */
  DSA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent          */
  DSA_ERR_DTYPE = 3,       /* dtype or dtype combination not provided         */
  DSA_ERR_ALIGN = 4,       /* a streamed / gathered array is not 16-B aligned */
  DSA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required         */
  DSA_ERR_UNSUPPORTED = 6, /* supported by the method, not by this library    */
  DSA_ERR_HIP = 7          /* the HIP runtime reported an error               */
} dsa_status;

typedef enum { DSA_F32 = 0, DSA_BF16 = 1, DSA_FP8_E4M3 = 2 } dsa_dtype;

/* Fixed row geometry of the absorbed MLA cache: 512 latent + 64 RoPE dims
 * ("GLM-5: from Vibe Coding...", section 2.1: a 576-dim latent KV cache;
 * "Zhipu AI / GLM", section 9.1: KV rank 512, 64 RoPE dims). */
#define DSA_LATENT_DIM 576
#define DSA_VALUE_DIM 512
/* Largest k this library selects (the pages use k = 2048 throughout). */
#define DSA_MAX_TOPK 2048
/* Most new tokens per sequence in one dsa_decode_fused step. */
#define DSA_MAX_TOKENS_PER_SEQ 8

/* Entry ids for dsa_workspace_size. */
#define DSA_ENTRY_INDEX_SCORES 0
#define DSA_ENTRY_TOPK 1
#define DSA_ENTRY_SPARSE_MLA 2
#define DSA_ENTRY_DECODE 3

/*
 * dsa_index_scores -- lightning-indexer scores.
 * The indexer scores every past key so the top-k can keep the important
 * tokens ("GLM-5: from Vibe Coding...", section 2.1.2: the lightning indexer
 * gives token-level sparsity; section 3.2: an extra indexer retrieves the
 * top-k key-value pairs; "Zhipu AI / GLM", section 9.1: DSA index 32 x 128).
 * The pages give no formula; this library computes the DeepSeek-V3.2 form
 *
 *   scores[r, s] = sum_h head_w[r, h] * ReLU( sum_d q_idx[r, h, d] * key_s[d] )
 *
 * for s = 0 .. q_pos[r], fp32 accumulation, fp32 result. Entries s > q_pos[r]
 * of a row are not written.
 *
 *   q_idx    [R, H_I, D_I]  q_dtype: DSA_BF16 or DSA_F32
 *   head_w   [R, H_I]       fp32
 *   k_idx    [cache_rows, D_I]  k_dtype: DSA_BF16 (with q BF16), DSA_FP8_E4M3
 *            (with q BF16; key = e4m3(code) * bf16(k_scale[row])), DSA_F32
 *            (with q F32). 16-B aligned.
 *   k_scale  [cache_rows] bf16 bits; required iff k_dtype == DSA_FP8_E4M3,
 *            otherwise ignored.
 *   row_off  [B] int64;  q_seq [R] int32 or NULL;  q_pos [R] int32
 *   H_I in 1..64, D_I in {64, 128}; max_n >= 1 bounds q_pos[r] + 1.
 *   scores   [R, ld_scores] fp32, ld_scores >= max_n, 16-B aligned rows
 *            (ld_scores % 4 == 0).
 */
dsa_status dsa_index_scores(const void* q_idx, int32_t q_dtype, const float* head_w,
                            const void* k_idx, int32_t k_dtype, const uint16_t* k_scale,
                            int64_t cache_rows, const int64_t* row_off, int32_t B,
                            const int32_t* q_seq, const int32_t* q_pos, int32_t R,
                            int32_t H_I, int32_t D_I, int32_t max_n,
                            float* scores, int64_t ld_scores, void* stream);

/*
 * dsa_index_scores_decode -- the indexer of dsa_decode_fused on its own: the
 * scores of B sequences with q_per_seq new tokens each, row r = b *
 * q_per_seq + i at position seq_len[b] - q_per_seq + i (the tokens' keys
 * already appended), as dsa_index_scores computes them for those rows. With
 * q_per_seq >= 2 each key row (bf16 or fp8) is read once for all of a
 * sequence's tokens (the multi-token step of dsa_decode_fused); paged caches
 * and rows over 2^22 keys use one key stream per token.
 *
 *   q_idx [R, H_I, D_I], head_w [R, H_I], R = B * q_per_seq;
 *   q_per_seq in 1 .. DSA_MAX_TOKENS_PER_SEQ
 *   seq_len [B] int32 (q_per_seq <= seq_len[b] <= max_len), row_off [B] int64
 *   scores [R, ld_scores] fp32, ld_scores >= max_len, % 4 == 0, 16-B aligned;
 *   entries past a row's position are left untouched
 * Other arguments, dtypes and errors as in dsa_index_scores.
 */
dsa_status dsa_index_scores_decode(const void* q_idx, int32_t q_dtype, const float* head_w,
                                   const void* k_idx, int32_t k_dtype, const uint16_t* k_scale,
                                   int64_t cache_rows, const int64_t* row_off,
                                   const int32_t* seq_len, int32_t B, int32_t q_per_seq,
                                   int32_t H_I, int32_t D_I, int32_t max_len, float* scores,
                                   int64_t ld_scores, void* stream);

/*
 * dsa_topk -- deterministic top-k over each score row.
 * k = 2048 ("Zhipu AI / GLM", sections 9.3 and 11.1). The selection must be
 * reproducible bit for bit: a non-deterministic top-k desynchronised
 * rollout and training and collapsed RL; the pages' fix is a deterministic
 * top-k ("GLM-5: from Vibe Coding...", section 3.2; "GLM-5 Notes", Replay).
 *
 * For row r with n = q_pos[r] + 1 candidates and k_eff = min(k, n):
 * idx_out[r, 0:k_eff] are the first k_eff keys of the stable descending
 * sort of scores[r, 0:n] (equal scores: lower key index first; -0.0 ranks
 * equal to +0.0), idx_out[r, k_eff:k] = -1. Selection and ordering are
 * integer operations on an order-preserving 32-bit image of each score, so
 * the result is unique and identical on every run. NaN scores are outside
 * the contract.
 *
 *   scores   [R, ld_scores] fp32, ld_scores % 4 == 0, 16-B aligned
 *   q_pos    [R] int32; max_n bounds q_pos[r] + 1 (host value)
 *   k        1 .. DSA_MAX_TOPK
 *   idx_out  [R, k] int32 (positions within the query's sequence)
 *   workspace: dsa_workspace_size(DSA_ENTRY_TOPK, ...) bytes (may be 0 -> NULL ok)
 */
dsa_status dsa_topk(const float* scores, int64_t ld_scores, const int32_t* q_pos,
                    int32_t R, int32_t max_n, int32_t k, int32_t* idx_out,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * dsa_sparse_mla_attn -- absorbed (MQA-form) MLA attention over the selected
 * keys only ("GLM-5: from Vibe Coding...", section 3.2: attention is computed
 * sparsely on the retrieved subset; section 2.1: 576-dim latent KV cache and
 * 576-dim dot products in decoding). One latent row per token is shared by all
 * heads; all 576 dims form the key, the first 512 the value:
 *
 *   l_j      = scale * q_abs[r, h, :] . latent[row(idx[r, j]), :]
 *   out[r,h] = sum_j softmax(l)_j * latent[row(idx[r, j]), 0:512]
 *   lse[r,h] = log sum_j exp(l_j)   (natural log)
 *
 * over the entries j < k with idx[r, j] >= 0 (-1 entries are skipped);
 * row(s) = row_off[q_seq[r]] + s. bf16/fp32 inputs, fp32 accumulation and
 * outputs. The key-split plan depends only on (R, H, k) and the device, so
 * the same indices give bitwise identical outputs (index replay: "GLM-5
 * Notes", Replay; "GLM-5: from Vibe Coding...", section 3.2).
 *
 *   q_abs    [R, H, 576]  dtype DSA_BF16 or DSA_F32
 *   latent   [cache_rows, 576], 16-B aligned, latent_dtype = dtype, or
 *            DSA_FP8_E4M3 with dtype DSA_BF16: OCP e4m3 codes (576 bytes per
 *            row) dequantised as code * latent_scale[row] (an FP8 KV cache,
 *            "Zhipu AI / GLM", section 11.4; one float32 scale per row is
 *            this library's reading). latent_scale [cache_rows] fp32, 4-B
 *            aligned, required for fp8 and ignored otherwise.
 *   idx      [R, k] int32;  k in 1 .. DSA_MAX_TOPK;  H in 1 .. 128;
 *            cache_rows < 2^31 (larger caches: DSA_ERR_UNSUPPORTED)
 *   out      [R, H, 512] fp32;  lse [R, H] fp32 or NULL
 *   workspace: dsa_workspace_size(DSA_ENTRY_SPARSE_MLA, R, 0, k, H) bytes
 * A row with no valid index gets out = 0 and lse = -inf.
 */
dsa_status dsa_sparse_mla_attn(const void* q_abs, int32_t dtype, const void* latent,
                               int32_t latent_dtype, const float* latent_scale,
                               int64_t cache_rows, const int64_t* row_off, int32_t B,
                               const int32_t* q_seq, const int32_t* idx, int32_t k,
                               int32_t R, int32_t H, float scale, float* out, float* lse,
                               void* workspace, size_t ws_bytes, void* stream);

/*
 * dsa_decode_fused -- one decode step: indexer -> top-k -> sparse MLA for B
 * sequences with q_per_seq new tokens each, their keys and latent rows
 * already appended. Query row r = b * q_per_seq + i is token i of sequence b,
 * at position seq_len[b] - q_per_seq + i, and selects its own top-k over its
 * own causal range. q_per_seq = 1 is plain decode; 2 .. 8 serves the tokens
 * of a multi-token (MTP / speculative) step ("GLM-5: from Vibe Coding...",
 * section 2.1: multi-token prediction with shared parameters, 4 speculative
 * steps; "Zhipu AI / GLM", section 11.1: MTP steps share top-k indices and
 * the KV cache). The indexer reads each key row (bf16 or fp8) once for all
 * of a sequence's new tokens (contiguous caches, rows up to 2^22 keys). Enqueues the same kernels as the three entry
 * points above, with the scores (and the indices when idx_out is NULL) kept
 * in the workspace; the attention split plan equals dsa_sparse_mla_attn's,
 * so replaying the recorded idx_out through dsa_sparse_mla_attn (q_seq[r] =
 * r / q_per_seq) reproduces out and lse bitwise.
 *
 *   R = B * q_per_seq;  q_per_seq in 1 .. DSA_MAX_TOKENS_PER_SEQ
 *   q_idx [R, H_I, D_I], head_w [R, H_I], k_idx/k_scale as in dsa_index_scores
 *   q_abs [R, H, 576], latent [cache_rows, 576]: act_dtype (DSA_BF16 or
 *   DSA_F32) is the dtype of q_idx and q_abs; latent_dtype and
 *   latent_scale as in dsa_sparse_mla_attn; k_dtype as in
 *   dsa_index_scores.
 *   seq_len [B] int32 (q_per_seq <= seq_len[b] <= max_len), row_off [B] int64
 *   out [R, H, 512] fp32, lse [R, H] or NULL, idx_out [R, k] int32 or NULL
 *   workspace: dsa_workspace_size(DSA_ENTRY_DECODE, R, max_len, k, H) bytes
 */
dsa_status dsa_decode_fused(const void* q_idx, const float* head_w, const void* k_idx,
                            int32_t k_dtype, const uint16_t* k_scale, const void* q_abs,
                            const void* latent, int32_t act_dtype, int32_t latent_dtype,
                            const float* latent_scale, int64_t cache_rows,
                            const int64_t* row_off, const int32_t* seq_len, int32_t B,
                            int32_t q_per_seq, int32_t max_len, int32_t H_I, int32_t D_I, int32_t H, int32_t k,
                            float scale, float* out, float* lse, int32_t* idx_out,
                            void* workspace, size_t ws_bytes, void* stream);

/*
 * dsa_decode_fused_noalloc -- dsa_decode_fused for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments, kernels and bits,
 * without workspace / ws_bytes. The workspace is a scratch array of the
 * library, dsa_decode_noalloc_limit() bytes (64 MiB) per device, held from
 * the first call on a device until the process ends; the call itself never
 * allocates or frees. A step whose workspace (dsa_workspace_size(
 * DSA_ENTRY_DECODE, ...)) exceeds the limit returns DSA_ERR_WORKSPACE
 * (dsa_last_error() names both sizes) before anything is enqueued. Nothing in
 * the scratch has to start at zero: every launch writes what it reads later.
 * All calls on one device share its scratch, so calls that overlap on one
 * GPU (concurrent streams, or several threads) race; serialise them.
 */
dsa_status dsa_decode_fused_noalloc(const void* q_idx, const float* head_w, const void* k_idx,
                                    int32_t k_dtype, const uint16_t* k_scale, const void* q_abs,
                                    const void* latent, int32_t act_dtype, int32_t latent_dtype,
                                    const float* latent_scale, int64_t cache_rows,
                                    const int64_t* row_off, const int32_t* seq_len, int32_t B,
                                    int32_t q_per_seq, int32_t max_len, int32_t H_I, int32_t D_I,
                                    int32_t H, int32_t k, float scale, float* out, float* lse,
                                    int32_t* idx_out, void* stream);

/* Bytes of scratch dsa_decode_fused_noalloc holds per device. */
size_t dsa_decode_noalloc_limit(void);

/*
 * Paged caches (the serving-engine layout: a pool of fixed-size pages and a
 * block table per sequence). Same computation and outputs as
 * dsa_sparse_mla_attn / dsa_decode_fused, with row_off replaced by:
 *   block_table [B, max_pages] int32: position s of sequence b is row
 *               s % page_size of page block_table[b][s / page_size], i.e.
 *               cache row block_table[b][s / page_size] * page_size +
 *               s % page_size of the indexer keys, their fp8 scales, the
 *               latent rows and their fp8 scales alike;
 *   page_size   a power of two in 64 .. 2^20 (DSA_ERR_UNSUPPORTED otherwise),
 *               cache_rows >= page_size; page ids outside the pool
 *               [0, cache_rows / page_size) are clamped into it;
 *   max_pages   >= 1; for the decode step max_pages * page_size >= max_len.
 * The computation per key does not depend on where the key is stored, so a
 * paged step gives the bits of the same step on a contiguous cache.
 * Several new tokens per sequence run with one key stream per token.
 */
dsa_status dsa_sparse_mla_attn_paged(const void* q_abs, int32_t dtype, const void* latent,
                                     int32_t latent_dtype, const float* latent_scale,
                                     int64_t cache_rows, const int32_t* block_table,
                                     int32_t max_pages, int32_t page_size, int32_t B,
                                     const int32_t* q_seq, const int32_t* idx, int32_t k,
                                     int32_t R, int32_t H, float scale, float* out, float* lse,
                                     void* workspace, size_t ws_bytes, void* stream);

dsa_status dsa_decode_fused_paged(const void* q_idx, const float* head_w, const void* k_idx,
                                  int32_t k_dtype, const uint16_t* k_scale, const void* q_abs,
                                  const void* latent, int32_t act_dtype, int32_t latent_dtype,
                                  const float* latent_scale, int64_t cache_rows,
                                  const int32_t* block_table, int32_t max_pages,
                                  int32_t page_size, const int32_t* seq_len, int32_t B,
                                  int32_t q_per_seq, int32_t max_len, int32_t H_I, int32_t D_I,
                                  int32_t H, int32_t k, float scale, float* out, float* lse,
                                  int32_t* idx_out, void* workspace, size_t ws_bytes,
                                  void* stream);

/*
 * Context parallelism over key ranges ("GLM-5: from Vibe Coding...", section
 * 2.4.2: long sequences split over context-parallel groups). Shard p holds
 * keys [lo_p, hi_p) of every sequence; it scores them (dsa_index_scores over
 * its cache rows, positions shifted by -lo_p), selects a local top-k
 * (dsa_topk) and turns it into a candidate list (dsa_topk_pairs); the
 * gathered lists [P, R, k] merge into the global top-k (dsa_topk_merge),
 * equal to the unsharded selection because the order (score descending,
 * lower key first) is total and the shards' keys are disjoint. Each shard
 * then attends over the global winners it holds (dsa_shard_indices, then
 * dsa_sparse_mla_attn) and the partial outputs merge by their log-sum-exp
 * in shard order (dsa_attn_merge), deterministic for a fixed P. On one
 * device the shards are views of one cache. All four only enqueue work on
 * `stream`; arguments are checked on the host.
 */

/* pair_score[r, j] = scores[r, idx[r, j]], pair_idx[r, j] = idx[r, j] +
 * key_offset (the shard's lo), -inf / -1 where idx[r, j] = -1.
 * scores [R, ld_scores] fp32; idx, pair_idx [R, k] int32; pair_score [R, k]. */
dsa_status dsa_topk_pairs(const float* scores, int64_t ld_scores, const int32_t* idx,
                          int32_t R, int32_t k, int32_t key_offset, float* pair_score,
                          int32_t* pair_idx, void* stream);

/* idx_out[r, :] = the first k of the union of the P lists pair_*[p, r, :]
 * (each in rank order with its -1 entries last, as dsa_topk_pairs leaves
 * them, keys disjoint across lists) in the order score descending, lower key
 * first; -1 past the candidates. pair_score [P, R, k] fp32, pair_idx
 * [P, R, k] int32; P in 1 .. 8 with P * k <= 16384 (else
 * DSA_ERR_UNSUPPORTED). Lists that break these rules give unspecified
 * indices (never an access outside the arrays). */
dsa_status dsa_topk_merge(const float* pair_score, const int32_t* pair_idx, int32_t P,
                          int32_t R, int32_t k, int32_t* idx_out, void* stream);

/* idx_local[r, j] = idx[r, j] - lo where lo <= idx[r, j] < hi, else -1:
 * the global winners a shard holds, in its own key numbering. [R, k] int32. */
dsa_status dsa_shard_indices(const int32_t* idx, int32_t R, int32_t k, int32_t lo, int32_t hi,
                             int32_t* idx_local, void* stream);

/* out[r, h] = sum_p exp(lse_p - LSE) o_p[r, h], lse[r, h] = LSE = log sum_p
 * exp(lse_p), summed in shard order; shards with lse -inf add nothing, and a
 * row with none gets out = 0, lse = -inf. P in 1 .. 8. o_parts [P, R, H, 512]
 * fp32 and out [R, H, 512] 16-B aligned; lse_parts [P, R, H]; lse [R, H] or NULL. */
dsa_status dsa_attn_merge(const float* o_parts, const float* lse_parts, int32_t P, int32_t R,
                          int32_t H, float* out, float* lse, void* stream);

/*
 * dsa_workspace_size -- bytes of workspace an entry point needs.
 * entry: one of DSA_ENTRY_*; rows = R (B * q_per_seq for DSA_ENTRY_DECODE);
 * max_len = longest sequence (decode) or max_n (top-k); k; H = MLA heads.
 * Returns 0 when the entry needs none; the result is a multiple of 256.
 * It queries the current device (the split plan depends on its CU count).
 */
size_t dsa_workspace_size(int32_t entry, int32_t rows, int32_t max_len, int32_t k, int32_t H);

/*
 * dsa_check_indices -- debug validator of index arrays: the structure the
 * top-k guarantees ("GLM-5 Notes", Replay: indices must be reproducible;
 * the entries are positions of selected keys), checked without the scores.
 * For query r with n = q_pos[r] + 1 and k_eff = min(k, n), an entry counts
 * as bad when, among the first k_eff, it lies outside [0, n) or repeats an
 * earlier valid one (each repeat counts once), or, past k_eff, it is not -1
 * (q_pos[r] < 0: every entry must be -1).
 * The count is ADDED to *n_bad (a device int32 the caller zeroes first; no
 * memset is enqueued, so the call may be captured in a graph).
 *
 *   idx   [R, k] int32 (device);  q_pos [R] int32 (device);  k in 1 .. DSA_MAX_TOPK
 *   n_bad device int32, accumulated with one atomic add per row with a bad entry
 * Enqueued on `stream`; returns DSA_ERR_NULL / DSA_ERR_SHAPE /
 * DSA_ERR_UNSUPPORTED for bad arguments before any launch.
 */
dsa_status dsa_check_indices(const int32_t* idx, const int32_t* q_pos, int32_t R, int32_t k,
                             int32_t* n_bad, void* stream);

/*
 * dsa_read_probe -- a measurement aid, no part of the method: a plain
 * streaming read of `bytes` bytes of device memory at `buf` (16-byte aligned,
 * bytes a positive multiple of 16), the attainable rate beside the published
 * HBM peak for a kernel that reads its operand once (the indexer's key stream
 * in "GLM-5: from Vibe Coding to Agentic Engineering", section 2.1.1: the
 * indexer scores every cached key once per query). One workgroup per CU
 * (dsa_read_probe_blocks() of them) reads the buffer in one contiguous sweep;
 * workgroup g writes the fp32 sum of the floats it read to out[g] (device,
 * out_len >= dsa_read_probe_blocks()), in an order that depends on the grid.
 * Enqueued on `stream`; DSA_ERR_NULL / DSA_ERR_SHAPE / DSA_ERR_ALIGN for bad
 * arguments before any launch.
 */
int32_t dsa_read_probe_blocks(void);
dsa_status dsa_read_probe(const void* buf, uint64_t bytes, float* out, int32_t out_len, void* stream);

/* Text of a status code (static storage). */
const char* dsa_status_string(int32_t status);

/* Text of the last DSA_ERR_HIP on the calling thread, or of the last
 * DSA_ERR_WORKSPACE of dsa_decode_fused_noalloc (static per thread). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
