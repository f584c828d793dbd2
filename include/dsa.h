/*
 * dsa.h — C ABI of the DSA sparse-attention layer on AMD Instinct MI355X (gfx950).
 *
 * The layer (one per MLA full-attention layer) runs, for every query row:
 *   1. the lightning indexer: score every visible cached token with 32 light heads over
 *      128-dim FP8 (or MXFP4) index keys                       -> dsa_indexer_scores
 *   2. an exact top-k select (k <= 2048)                      -> dsa_topk
 *   3. exact MLA attention of all 96 heads over only the selected latents
 *                                                              -> sparse_mla_decode / _prefill
 * Source: "vLLM Delivers Day-0 Support for Kimi K3.1 Pro" (§Sparse Attention in K3.1 Pro for the
 * three steps and the 132-byte FP8 index key / 576-byte FP8 latent; §A KV cache for three kinds
 * of state for the block-packed paged cache, its power-of-two block size, the NVFP4 latent and
 * MXFP4 index-key variants, and block tables translated into kernel-page addresses; §Low-latency
 * decode for the scorer + exact select that hands attention the physical KV rows;
 * §AMD / Quantization: Native MXFP4 indexer for 68-byte MXFP4 keys scored on FP4 matrix
 * instructions with FP32 accumulation).  The scoring rule is the DeepSeek-V3.2 lightning
 * indexer's, to which the page defers:
 *     score[r,s] = sum_h w[r,h] * ReLU(scale_s * q[r,h] . k[s]).
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless the comment says "host".  The caller owns every
 *     buffer (pool, tables, queries, outputs, workspaces); the library never allocates or frees
 *     device memory and never synchronises (dsa_device_status alone waits for its stream): work
 *     is enqueued on `stream` (a hipStream_t of the current device; NULL is the default stream)
 *     and buffers must stay valid until it completes.
 *   - Errors are returned, never thrown.  Host-side validation runs before anything is launched;
 *     a failed call launches nothing.  dsa_last_error() gives a per-thread message.
 *   - Device data that breaks the contract is detected where it is read and recorded in a
 *     per-device status word (DSA_DEVERR_* bits below; dsa_device_status reads and clears it):
 *     a block-table entry outside the pool (the scorer scores that block's tokens as 0, the
 *     attention skips them), a pool row past the pool given to the attention (skipped), a
 *     sequence with more rows than max_rows_per_seq (its extra rows are not scored).  Selected
 *     indices outside [0, row position] are ignored by the attention (-1 is the padding).
 *   - Identical inputs give bit-identical outputs.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifndef DSA_API
#define DSA_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned buffer, k out of range, ... */
  DSA_ERR_UNSUPPORTED = 2, /* a format or shape this build does not implement */
  DSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the *_workspace_bytes query */
  DSA_ERR_HIP = 4          /* a HIP runtime call failed; dsa_last_error() has its text */
} dsa_status;

/* Index-key formats (page: FP8 keys of 132 B/token incl. scale; opt-in MXFP4 keys, 68 B). */
enum { DSA_IKEY_FP8 = 0, DSA_IKEY_MXFP4 = 1 };
/* Latent formats (page: FP8 latent, 576 B/token; NVFP4 latent). */
enum { DSA_LATENT_FP8 = 0, DSA_LATENT_NVFP4 = 1 };

/* Fixed model geometry (page: 32 indexer heads x 128 dims, top-2048, 96 attention heads; the
 * MLA latent is 576 wide and its first 512 dims are the value). */
enum {
  DSA_INDEX_HEADS = 32,
  DSA_INDEX_DIM = 128,
  DSA_MLA_HEADS = 96,
  DSA_MLA_DQK = 576,
  DSA_MLA_DV = 512,
  DSA_MAX_TOPK = 2048,
  DSA_HIST_BINS = 2048,
  DSA_MAX_ROWS_PER_SEQ = 8
};

/*
 * Paged, block-packed KV pool (one layer).  The pool is num_blocks rows of row_bytes bytes; row
 * b holds tokens [0, block_size) of whichever block the block tables map to b.  Inside a row
 * the pages are structure-of-arrays, each starting 16-byte aligned at the given byte offset:
 *   latent_format FP8:    latent       [bs][576] E4M3        at latent_off
 *                         latent scale [bs] fp32             at latent_scale_off
 *   latent_format NVFP4:  latent       [bs][288] packed E2M1 at latent_off  (element 2j is the
 *                                                            low nibble of byte j)
 *                         block scales [bs][36] E4M3 (one per 16 elements) at latent_scale_off
 *                         value = E2M1 * block scale * latent_tensor_scale
 *   ikey_format FP8:      keys         [bs][128] E4M3        at ikey_off, in the scorer's load
 *                         order: byte b of slot t at 2048 (t / 16) + 1024 (b / 64)
 *                         + 256 ((b / 16) % 4) + 16 (t % 16) + b % 16 (each 16-byte piece a
 *                         64-lane load takes, one per lane, is then part of one 1 KB run)
 *                         key scale    [bs] fp32 (> 0)       at ikey_scale_off
 *   ikey_format MXFP4:    keys         [bs][64] packed E2M1  at ikey_off
 *                         block scales [bs][4] E8M0 (one per 32 elements) at ikey_scale_off
 * row_bytes is a multiple of 256, and every page lies inside the row; the latent-scale page must
 * also have at least 12 bytes of the row behind it (the attention copies a token's latent scales
 * as whole 16-byte pieces).  Entry points reject a layout that breaks these rules with
 * DSA_ERR_INVALID_ARG; dsa_kv_layout_init always meets them.  Token s of a sequence lives in row
 * block_table[s / bs], slot s % bs; its physical row index is block_table[s / bs] * bs + s % bs.
 */
typedef struct dsa_kv_layout {
  int32_t block_size;    /* tokens per block; this build supports 64 */
  int32_t ikey_format;   /* DSA_IKEY_* */
  int32_t latent_format; /* DSA_LATENT_* */
  int32_t reserved;
  int64_t row_bytes;
  int64_t latent_off, latent_scale_off, ikey_off, ikey_scale_off;
  int64_t num_blocks;        /* rows in the pool */
  float latent_tensor_scale; /* NVFP4 only: the fp32 tensor scale (> 0); 1 otherwise */
} dsa_kv_layout;

/*
 * Query rows of one call, grouped by sequence.  Row r sits at absolute position row_pos[r] and
 * sees tokens [0, row_pos[r]] of its sequence (its own token included: the new token's key and
 * latent are in the cache before the layer runs).  Several rows of one sequence (speculative
 * verification, chunked prefill) read that sequence's keys once.
 */
typedef struct dsa_batch {
  int32_t num_seqs;
  int32_t num_rows;
  int32_t max_rows_per_seq;   /* host: upper bound on rows of any one sequence (>= 1; 0 only
                                 when num_rows is 0: every entry point then returns DSA_OK
                                 and launches nothing) */
  int32_t max_blocks_per_seq; /* host: leading dimension of block_table */
  int64_t max_context;        /* host: upper bound on row_pos[r] + 1 over all rows */
  const int32_t* block_table;   /* [num_seqs * max_blocks_per_seq] pool row ids */
  const int32_t* seq_row_start; /* [num_seqs + 1] rows of sequence b: [start[b], start[b+1]) */
  const int32_t* row_pos;       /* [num_rows] */
  uint32_t flags;               /* host: DSA_BATCH_* bits below (any other bit: INVALID_ARG) */
} dsa_batch;

/* dsa_batch.flags: the attention splits each row's selected set into fixed 128-token parts, in
 * sparse_mla_decode and sparse_mla_prefill alike, so a row's outputs are bit-identical whichever
 * rows share its batch and whichever of the two runs it (the page's batch-invariant kernels).
 * Without it the split count follows the row count (faster; outputs then agree within rounding
 * between batches of different row counts).  Scores and the select are batch-invariant always. */
#define DSA_BATCH_INVARIANT 1u

/* dsa_batch.flags: score the row tiles of a prefill chunk in plain ascending order.  By default
 * they are dispatched in the balanced order of token-sharded prefill (§Prefill: shard the attention
 * by token, not by head): the chunk's row tiles are cut into 16 contiguous pieces and slot
 * s = 0..7 takes pieces s and 15 - s, so that under the causal mask each stretch of dispatched
 * work pairs a light piece with a heavy one.  Results are identical either way. */
#define DSA_BATCH_PLAIN_ORDER 2u

/* Bits of the device status word.  Once set, a bit stays set until dsa_device_status clears it;
 * while DSA_DEVERR_ROWS_PER_SEQ is set, every dsa_topk on that device writes count = -1 and
 * idx = phys = -1 for all of its rows (the rows a scorer skipped have no scores to select from). */
#define DSA_DEVERR_ROWS_PER_SEQ 1u /* a sequence had more rows than dsa_batch.max_rows_per_seq */
#define DSA_DEVERR_BLOCK_ID 2u     /* a block-table entry of a visible block was outside the pool */
#define DSA_DEVERR_POOL_ROW 4u     /* a physical row given to the attention was past the pool */
#define DSA_DEVERR_CAND_OVERFLOW 8u /* a row's candidate list outgrew its capacity (candidates path) */

/* Fill *out (host) with the pool layout for the given formats (block_size must be 64).
 * Returns INVALID_ARG for a null pointer or bad value, UNSUPPORTED for another block size. */
DSA_API dsa_status dsa_kv_layout_init(dsa_kv_layout* out, int32_t ikey_format, int32_t latent_format,
                              int32_t block_size, int64_t num_blocks, float latent_tensor_scale);

/*
 * Step 1 — lightning-indexer scores of every visible token, for every row.
 *   q_idx  [num_rows][32][128] E4M3 indexer queries (any quantisation scale folded into w)
 *   w      [num_rows][32] fp32 head weights
 *   scores [num_rows][ld_scores] fp32 output; entries [0, row_pos[r]] are written, the rest are
 *          left untouched.  ld_scores >= max_context.
 *   hist   [num_rows][DSA_HIST_BINS] uint32 in/out or NULL (4-byte aligned): counts of the top
 *          11 bits of each written score's order-preserving key are added to it; dsa_topk
 *          consumes it (saving a pass over the scores) and returns it to zero.  It must be all
 *          zero on entry: allocate it zeroed once, and clear it yourself if scores are computed
 *          without a dsa_topk call.  Without it dsa_topk builds the counts in a pass of its own.
 * Decode and speculative decode (max_rows_per_seq <= DSA_MAX_ROWS_PER_SEQ) stream the index keys
 * once per sequence and score all of that sequence's rows from each key read.  Prefill chunks
 * (more rows per sequence; FP8 or MXFP4 keys) score tiles of 16 rows, streaming each key page once
 * per tile.
 * Exactness: key products are exact and accumulate in fp32; scale_s > 0 is applied after the
 * head sum (equal to applying it inside each ReLU whenever the sums are exact).
 */
DSA_API dsa_status dsa_indexer_scores(const dsa_kv_layout* kv, const void* pool, const dsa_batch* batch,
                              const uint8_t* q_idx, const float* w, float* scores,
                              int64_t ld_scores, uint32_t* hist, void* stream);

/* Workspace bytes dsa_topk needs for num_rows rows whose positions are below max_context. */
DSA_API size_t dsa_topk_workspace_bytes(int32_t num_rows, int64_t max_context);

/*
 * Step 2 — exact top-k per row (page: keep the 2,048 highest-scoring tokens).  Order: score
 * descending, token index ascending (a tie goes to the lower index); -0 equals +0.  NaN scores
 * are not supported.
 *   scores/ld_scores/hist as produced by step 1 (hist may be NULL: the histogram is then built
 *         here, one more pass over the scores).  A given hist is returned to zero.
 *   k in [1, DSA_MAX_TOPK]; max_context up to 8,388,608
 *   idx   [num_rows][k] int32 output: the selected token indices in ascending order, then -1
 *   count [num_rows] int32 output: min(k, row_pos[r] + 1)
 *   phys  [num_rows][k] int32 output or NULL: physical pool rows (block * bs + slot) of idx,
 *         -1 padded (kv is required when phys is not NULL)
 *   workspace: device scratch of at least dsa_topk_workspace_bytes(num_rows, max_context) bytes
 */
DSA_API dsa_status dsa_topk(const dsa_kv_layout* kv, const dsa_batch* batch, const float* scores,
                            int64_t ld_scores, uint32_t* hist, int32_t k, int32_t* idx,
                            int32_t* count, int32_t* phys, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Steps 1 and 2 without stored scores: the candidates path (page: two kernels, a scorer and then an
 * exact top-k select, §Low-latency decode: a fused DSA decode path).  The scores of a full row
 * are never written; the select receives only the tokens that can still make the row's top-k.
 *   dsa_indexer_candidates  scores a sample of each sequence (every S-th 64-token block, S a power
 *       of two near sqrt(max_context / 2k), chosen by the library), takes the sample's exact
 *       top-k per row (kept as the row's first candidates) and its k-th key T with the tie cutoff
 *       I, then scores the other blocks and keeps each token whose key (the order-preserving image
 *       of its score) is above T, or equal to T with an index below I.  Any other token is beaten
 *       by k sample tokens, so the candidates contain the exact top-k.
 *   dsa_topk_candidates     selects each row's top-k from its candidates: the same result as
 *       dsa_topk on dense scores (idx ascending, -1 padded; count; phys as in dsa_topk).
 * Both take the same batch, k and workspace (at least dsa_candidates_workspace_bytes(num_rows,
 * batch->max_context, k) bytes, 16-byte aligned; nothing in it has to be initialised), and the
 * second must follow the first on the stream.  Limits: max_context up to 8,388,608; k in
 * [1, DSA_MAX_TOPK].  A row's candidate list holds 2 S (k + 64) + k entries (about twice what
 * independent scores produce); a row whose candidates outgrow it (scores far above the sample's
 * in the blocks that were not sampled) gets count = -1 and idx = phys = -1, and the status word
 * gets DSA_DEVERR_CAND_OVERFLOW: rerun such rows on the dense path (dsa_indexer_scores +
 * dsa_topk), which is exact for every input.  While DSA_DEVERR_ROWS_PER_SEQ is set,
 * dsa_topk_candidates writes count = -1 for every row, as dsa_topk does.
 */
DSA_API size_t dsa_candidates_workspace_bytes(int32_t num_rows, int64_t max_context, int32_t k);
DSA_API dsa_status dsa_indexer_candidates(const dsa_kv_layout* kv, const void* pool,
                                          const dsa_batch* batch, const uint8_t* q_idx,
                                          const float* w, int32_t k, void* workspace,
                                          size_t workspace_bytes, void* stream);
DSA_API dsa_status dsa_topk_candidates(const dsa_kv_layout* kv, const dsa_batch* batch, int32_t k,
                                       void* workspace, size_t workspace_bytes, int32_t* idx,
                                       int32_t* count, int32_t* phys, void* stream);

/* Workspace bytes sparse_mla_decode needs for num_rows rows and top-k k with dsa_batch.flags
 * `flags` (sparse_mla_prefill needs none unless flags has DSA_BATCH_INVARIANT: then this size). */
DSA_API size_t sparse_mla_workspace_bytes(int32_t num_rows, int32_t k, uint32_t flags);

/*
 * Step 3 — exact MLA attention over the selected latents (page: attention is exact but limited
 * to the chosen tokens, for all heads; the latent is shared by all heads).  For row r and
 * head h, over j in idx[r][0..k) with idx >= 0:
 *   c_j = dequantised latent of token idx[r][j] (FP8 code * token scale, or NVFP4)
 *   logit_j = softmax_scale * q[r,h] . c_j ;  p = softmax(logit)
 *   out[r,h] = sum_j p_j c_j[0:512] ;  lse[r,h] = max + ln sum exp(logit - max)
 *   q    [num_rows][96][576] bf16;  idx [num_rows][k] from dsa_topk
 *   phys [num_rows][k] pool rows of idx from dsa_topk, or NULL (then idx is translated through
 *        the block table here).  Passing the rows the select already emitted saves a dependent
 *        lookup per token (page: the select hands the attention pool rows, not logical indices).
 *   out  [num_rows][96][512] bf16 output;  lse [num_rows][96] fp32 output or NULL
 *   workspace: device scratch of at least sparse_mla_workspace_bytes(num_rows, k) bytes
 * A row with no selected token gets out = 0 and lse = -inf.  Latent token scales (FP8) and the
 * tensor scale (NVFP4) must be positive and below 4096 (they scale fp16 probabilities).
 * The decode variant splits each row's selected set over several workgroups and merges the
 * partial results by log-sum-exp; the prefill variant (for thousands of rows) gives each row one
 * workgroup across all heads and needs no workspace (it may be NULL).
 */
DSA_API dsa_status sparse_mla_decode(const dsa_kv_layout* kv, const void* pool, const dsa_batch* batch,
                             const uint16_t* q, const int32_t* idx, const int32_t* phys, int32_t k,
                             float softmax_scale, uint16_t* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);
DSA_API dsa_status sparse_mla_prefill(const dsa_kv_layout* kv, const void* pool, const dsa_batch* batch,
                              const uint16_t* q, const int32_t* idx, const int32_t* phys, int32_t k,
                              float softmax_scale, uint16_t* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * sparse_mla_decode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels and results,
 * bit for bit, but the split partials live in a static 64 MiB array the library holds in each
 * device's memory until the process ends, so the call takes no workspace and allocates nothing.
 * Arguments as sparse_mla_decode.  Limit: sparse_mla_workspace_bytes(num_rows, k, flags) must be
 * at most 64 MiB (every batch of up to 135 rows at k = 2,048; up to 42 rows with
 * DSA_BATCH_INVARIANT), else DSA_ERR_WORKSPACE, checked before anything is launched.  Nothing in
 * the array has to start at zero.  All calls on one device share that array: calls that overlap in time on
 * one device (other streams, other threads) race and must be ordered by the caller.  The stream
 * must belong to the current device.
 */
DSA_API dsa_status sparse_mla_decode_noalloc(const dsa_kv_layout* kv, const void* pool,
                                             const dsa_batch* batch, const uint16_t* q,
                                             const int32_t* idx, const int32_t* phys, int32_t k,
                                             float softmax_scale, uint16_t* out, float* lse,
                                             void* stream);

/*
 * The step before the path ("vLLM Delivers Day-0 Support for Kimi K3.1 Pro", §Low-latency decode:
 * a fused DSA decode path: the indexer query is quantised with the head weights merged into its
 * scale, and the appended token's index key and latent go into the KV cache, the latent write
 * overlapping the indexer).  Rounding is to the nearest code, ties to the even code, saturating at the format's
 * largest finite value; inputs must be finite.  The codes are exact functions of the bf16 inputs.
 *
 * dsa_cache_append — quantise num_tokens new tokens into their pool rows (formats as in
 * dsa_kv_layout):
 *   FP8 index key / FP8 latent: per-token scale amax / 448 (1 when amax is 0), codes E4M3(x / s)
 *   MXFP4 index key: per 32 elements E8M0 exponent floor(log2 amax) - 2 (127 when amax is 0),
 *     codes E2M1(x / 2^(E-127))
 *   NVFP4 latent: per 16 elements block scale E4M3((amax / 6) / tensor scale), codes
 *     E2M1(x / (block scale * tensor scale)) (0 when that product is 0)
 *   slot      [num_tokens] int64 physical pool rows (block * block_size + slot in block, the
 *             numbering of dsa_topk's phys); a negative entry or one >= num_blocks * block_size
 *             is skipped (nothing written)
 *   index_key [num_tokens][128] bf16 or NULL (keys not written);  latent [num_tokens][576] bf16
 *             or NULL (latents not written): a caller can write the keys before the scorer and
 *             the latents on another stream while it runs
 * Two entries naming one slot race.  Returns INVALID_ARG for a bad layout, pointer or alignment
 * (slot 8-byte, index_key 4-byte, latent 8-byte aligned).
 */
DSA_API dsa_status dsa_cache_append(const dsa_kv_layout* kv, void* pool, int32_t num_tokens,
                                    const int64_t* slot, const uint16_t* index_key,
                                    const uint16_t* latent, void* stream);

/*
 * dsa_quantize_query — the indexer query in the form dsa_indexer_scores reads: per row r and
 * head h, s = amax_h / 448 (1 when amax_h is 0), q_idx[r][h] = E4M3(q[r][h] / s) and
 * w_out[r][h] = w[r][h] * s (so w_out ReLU(q_idx . k) = w ReLU(s q_idx . k)).
 *   q [num_rows][32][128] bf16 (4-byte aligned);  w [num_rows][32] fp32
 *   q_idx [num_rows][32][128] E4M3 output (2-byte aligned);  w_out [num_rows][32] fp32 output
 *   (w_out may be w)
 */
DSA_API dsa_status dsa_quantize_query(int32_t num_rows, const uint16_t* q, const float* w,
                                      uint8_t* q_idx, float* w_out, void* stream);

/*
 * dsa_indexer_front — what the scorer needs before it runs, in one launch: the new tokens' index
 * keys into their pool rows, as dsa_cache_append with latent = NULL, and the indexer query, as
 * dsa_quantize_query.  The results are bit-identical to those two calls.  The latents are left to
 * a dsa_cache_append(index_key = NULL) call, which can run on another stream while the scorer
 * runs, since the scorer reads no latent.
 *   slot, index_key  as in dsa_cache_append (may be NULL when num_tokens is 0)
 *   q, w, q_idx, w_out  as in dsa_quantize_query (may be NULL when num_rows is 0; w_out may be w)
 * Returns INVALID_ARG for a bad layout, a negative count, a missing pointer or a misalignment
 * (the alignments of the two calls); OK without a launch when both counts are 0.
 */
DSA_API dsa_status dsa_indexer_front(const dsa_kv_layout* kv, void* pool, int32_t num_tokens,
                                     const int64_t* slot, const uint16_t* index_key,
                                     int32_t num_rows, const uint16_t* q, const float* w,
                                     uint8_t* q_idx, float* w_out, void* stream);

/*
 * Decode context parallelism, emulated on one GPU ("vLLM Delivers Day-0 Support for Kimi K3.1
 * Pro", §Long context: decode context parallelism with a sparse indexer; §An exact top-k merge with
 * 10x less traffic; §AMD / Communication: Efficient cross-GPU communication).  Shard r of W holds
 * tokens r, r + W, r + 2W, ... of each sequence in a pool of its own (token j of the shard is
 * token j W + r of the sequence); a row at position p sees the shard's tokens [0, (p - r) / W].
 * One layer step: per shard, dsa_indexer_scores and dsa_topk (k) on that shard, then
 * dsa_dcp_publish; then dsa_dcp_merge once (every shard would run the same select on the same
 * gathered messages); then, per shard, sparse_mla_decode_shard over its part of the selection
 * (shard_idx[r]); then dsa_lse_combine.  The selected set equals the top-k of the whole sequence
 * (score descending, token index ascending) exactly, in every message variant.
 *
 * Message variants of the merge (what each shard sends per row):
 *   DSA_MERGE_PACKED  its best min(k, ceil(1.5 k / W)) candidates, 32 bits each: the upper 16 bits
 *                     of the score's order-preserving key and the candidate's 16-bit rank in its
 *                     own list (the page's packed candidates)
 *   DSA_MERGE_SCORES  its whole local top-k as fp32 scores; token indices stay local (the AMD
 *                     section's score-only exchange)
 *   DSA_MERGE_GENERIC its whole local top-k as (fp32 score, index) pairs (the generic merge)
 * The select finds the k-th largest message key.  A shard that sent fewer candidates than it holds
 * and whose weakest sent candidate reaches that threshold resends its full local top-k, and the
 * select is redone (at most once).  Entries equal to the threshold key, when only some of them are
 * needed, are ordered exactly by (score, index) from a second small exchange of their score and
 * index.
 */
enum { DSA_MERGE_PACKED = 0, DSA_MERGE_SCORES = 1, DSA_MERGE_GENERIC = 2, DSA_MAX_SHARDS = 8 };

/* Bytes of the mailbox (the exchange buffer the shards' lists go to) for num_rows rows, top-k k
 * and num_shards shards (0 for an out-of-range argument). */
DSA_API size_t dsa_dcp_mailbox_bytes(int32_t num_rows, int32_t k, int32_t num_shards);

/* Shard `shard` publishes each row's local top-k, sorted by score descending and local index
 * ascending, with global token indices (local * num_shards + shard).
 *   scores/ld_scores: that shard's dsa_indexer_scores output;  idx/count: its dsa_topk output (k)
 *   mailbox: at least dsa_dcp_mailbox_bytes(num_rows, k, num_shards) bytes, 16-byte aligned; the
 *   calls for all shards (any order) must complete before dsa_dcp_merge reads it. */
DSA_API dsa_status dsa_dcp_publish(int32_t num_rows, int32_t k, int32_t num_shards, int32_t shard,
                                   const float* scores, int64_t ld_scores, const int32_t* idx,
                                   const int32_t* count, void* mailbox, size_t mailbox_bytes,
                                   void* stream);

/* The exact merge.  Outputs:
 *   idx   [num_rows][k] global token indices ascending, then -1;  count [num_rows]
 *   shard_idx   [num_shards][num_rows][k] each shard's selected LOCAL indices ascending, then -1
 *               (the idx argument of that shard's sparse_mla_decode);  shard_count [num_shards][num_rows]
 *   stats [num_rows][4] or NULL: rounds (1, or 2 after a resend), shards that resent, entries of
 *         the tie exchange (0 if none), bytes all shards sent for the row over all rounds. */
DSA_API dsa_status dsa_dcp_merge(int32_t num_rows, int32_t k, int32_t num_shards, int32_t variant,
                                 void* mailbox, size_t mailbox_bytes, int32_t* idx, int32_t* count,
                                 int32_t* shard_idx, int32_t* shard_count, int32_t* stats,
                                 void* stream);

/* Bytes of the partials buffer that sparse_mla_decode_shard fills and dsa_lse_combine reads, for
 * num_rows rows, top-k k, num_shards shards and dsa_batch.flags `flags` (0 for a bad argument). */
DSA_API size_t dsa_dcp_partials_bytes(int32_t num_rows, int32_t k, int32_t num_shards,
                                      uint32_t flags);

/* One shard's attention over its part of the selection (idx = that shard's shard_idx, local
 * indices; count = its shard_count, or NULL; kv/pool/batch: the shard's own pool and batch; phys
 * NULL, or the shard's pool rows).  Arguments as sparse_mla_decode, except that nothing is written
 * to an output: the row's splits (fp16 outputs normalised and scaled by a power of two per head,
 * with their base-2 LSE) go to the shard's slots of `partials`, so the calls of all shards (in any
 * order) fill the buffer for one dsa_lse_combine.  The shard's split count is sized for k /
 * num_shards tokens; with count, each row's count entries are spread evenly over the splits (no
 * split walks the -1 tail), without it the splits cover all k slots. */
DSA_API dsa_status sparse_mla_decode_shard(const dsa_kv_layout* kv, const void* pool,
                                           const dsa_batch* batch, const uint16_t* q,
                                           const int32_t* idx, const int32_t* count,
                                           const int32_t* phys, int32_t k,
                                           float softmax_scale, int32_t shard, int32_t num_shards,
                                           void* partials, size_t partials_bytes, void* stream);

/* Log-sum-exp merge of all shards' partial attention results (page: partial outputs combined by
 * their LSE): for each row and head, over every split slot s of every shard with LSE l_s (natural
 * log here), M = max l_s, out = sum_s e^(l_s - M) o_s / sum_s e^(l_s - M) (bf16, fp32
 * accumulation in slot order), lse = M + ln(sum_s e^(l_s - M)); out = 0 and lse = -inf where no
 * shard selected a token.  k, num_shards and flags must be those of the shard calls; lse may be
 * NULL.  The exchanged partials take as many bytes as bf16 outputs but keep 11 significant bits
 * relative to the head's largest value, so the merged output keeps the single-GPU precision. */
DSA_API dsa_status dsa_lse_combine(int32_t num_rows, int32_t k, int32_t num_shards, uint32_t flags,
                                   const void* partials, size_t partials_bytes, uint16_t* out,
                                   float* lse, void* stream);

/* Measurement only (computes nothing of the method): stream num_pages pages of bytes_per_page
 * bytes each, page i at base + (rows ? rows[i] : i) * row_bytes + offset, with no arithmetic
 * behind the loads, on `grid` workgroups that each leave one word (the XOR of what they read) in
 * sink[grid].  With rows = the physical blocks a scorer visits and offset = the key page, this is
 * the ceiling of the scorer's access pattern; with rows = NULL and row_bytes = bytes_per_page, a
 * contiguous read.  bytes_per_page: a multiple of 16 up to 9,216; base + offset and row_bytes
 * 16-byte aligned; grid in [1, 65535].  Every page must lie in memory the caller owns. */
DSA_API dsa_status dsa_probe_read(const void* base, int64_t row_bytes, int64_t offset,
                                  int32_t bytes_per_page, const int32_t* rows, int64_t num_pages,
                                  uint32_t* sink, int32_t grid, void* stream);

/* The status word of the current device (DSA_DEVERR_* bits, 0 when every call so far met its
 * contract).  This call synchronises `stream` (which must belong to the current device) before
 * reading, so the word covers all work enqueued on it; clear != 0 then resets the word to 0.
 * Work on other streams that is still running may set bits after the read. */
DSA_API dsa_status dsa_device_status(uint32_t* status, int32_t clear, void* stream);

/* Text of a status code, and the calling thread's last error message ("" if none). */
DSA_API const char* dsa_status_string(dsa_status s);
DSA_API const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
