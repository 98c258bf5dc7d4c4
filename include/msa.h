/*
 * msa.h -- C ABI of the MI355X (gfx950) MiniMax Sparse Attention hot path.
 *
 * Two stages, after the pages:
 *   index branch  -- a single-head index key is max-pooled per KV block, each
 *                    query's index vector is scored against those summaries,
 *                    and each query keeps its causal top-K blocks
 *                    ([YLY] paragraph "索引分支（Index Branch）");
 *   sparse branch -- standard GQA over the selected blocks only
 *                    ([YLY] paragraph "稀疏分支（Sparse Branch）"), organised
 *                    as "KV outer, gather Q": each KV block is read once and
 *                    applied to every query that chose it
 *                    ([CXT] section 2.2 "KV Outer Gather Q：MSA 的关键设计"),
 *                    with per-block partial outputs merged by log-sum-exp.
 * Pages:
 *   [YLY] "MiniMax M3模型算力成本大幅降低原因深度解析",
 *         youleyou.com/wenzhang/3016623.html
 *   [CXT] "MiniMax M3 深度实战：当稀疏注意力打破百万 Token 墙 ...",
 *         chenxutan.com/d/3746.html
 *
 * Conventions for every call
 *   - Tensor pointers are DEVICE pointers to dense row-major arrays owned by
 *     the caller.  The library never allocates, frees or keeps caller memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work on it and return at once.
 *   - Return value: MSA_OK, or a negative msa_status.  Arguments are checked
 *     before anything is enqueued; on an error nothing is enqueued and no
 *     output is touched.  MSA_ERR_HIP reports a failed launch.  Faults inside
 *     kernels surface at the caller's next synchronisation, not here.
 *   - Outputs are fully overwritten (no pre-zeroing needed) unless a call
 *     says otherwise.  Workspaces are scratch: their contents on entry do not
 *     matter and are undefined on exit.
 *   - Inputs must be finite.  Calls on one stream are ordered; calls that
 *     share a workspace must not overlap.  No global mutable state except
 *     msa_decode_step_noalloc's per-device scratch (see there): every other
 *     call is safe from several host threads.
 *   - Block size B: a multiple of 16, at most 4096.  Top-K: 1 <= K <= 64.
 *     Index dimension d_idx: 1..1024 (multiples of 4 up to 1024, any value up
 *     to 256).  Token positions and counts are at most 2^40, Hq at most
 *     65536 and d at most 1024; a shape whose workspace would reach 2^60
 *     bytes is refused (MSA_ERR_INVALID_ARG, and its size query returns 0).
 *   - Positions count from 0.  own(p) = p / B is a token's own block.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent shapes */
  MSA_ERR_UNSUPPORTED = -2, /* no kernel built for this (dtype, d, B, ...)  */
  MSA_ERR_WORKSPACE = -3,   /* workspace smaller than the size query says  */
  MSA_ERR_HIP = -4          /* a HIP launch or runtime call failed         */
} msa_status;

typedef enum { MSA_F32 = 0, MSA_BF16 = 1, MSA_FP8_E4M3 = 2 } msa_dtype;
/* MSA_FP8_E4M3 (OCP e4m3: 4 exponent bits, bias 7, 3 mantissa bits, no
 * infinities) is accepted only as the KV dtype of msa_sparse_gqa_decode_paged. */

/* Human-readable name of a status code (static storage, never NULL). */
const char *msa_status_string(int status);

/* --------------------------------------------------------------------------
 * msa_index_pool -- block max-pool of index keys.  [YLY] "索引分支（Index Branch）"
 *
 *   kmax[s][b][c] = max over t in [b*B, min(b*B+B, len_s)) of idx_k[s][t][c]
 *
 * for every sequence s and every block b of the requested range that holds
 * at least one valid token (b*B < len_s); other entries of kmax are left
 * untouched.  The max is exact and uses the total order -0 < +0.
 *
 *   idx_k    [n_seq][len_max][d_idx] fp32
 *   seq_len  device int64 [n_seq], 1 <= len_s <= len_max; NULL = all len_max
 *   blocks   [blk_begin, blk_end) with 0 <= blk_begin < blk_end <= nb_max;
 *            blk_begin == -1 selects, per sequence, only the block holding its
 *            last token (len_s - 1) / B -- the block a decode step appends to
 *            -- and re-pools it from all its tokens;
 *            blk_begin == -2 is the O(d_idx) append form of the same update:
 *            with t = len_s - 1, kmax[s][t/B] = idx_k[s][t] when t starts the
 *            block, else max(kmax[s][t/B], idx_k[s][t]).  It is exact provided
 *            kmax[s][t/B] already holds the max over tokens [t/B*B, t), which
 *            holds after a full pool or a previous append of token t-1.
 *            blk_end is ignored for both modes.
 *   kmax     [n_seq][nb_max][d_idx] fp32, nb_max >= ceil(len_max / B)
 * ------------------------------------------------------------------------ */
int msa_index_pool(const float *idx_k, int32_t n_seq, int64_t len_max,
                   const int64_t *seq_len, int32_t d_idx, int32_t block,
                   int64_t blk_begin, int64_t blk_end, float *kmax,
                   int64_t nb_max, void *stream);

/* --------------------------------------------------------------------------
 * msa_index_pool_mean -- block mean-pool of index keys, a variant of the
 * summary for ablations: [CXT] section 3.3's sketch summarises a key block
 * by the mean over its tokens (instead of the max-pool the index branch of
 * [YLY] uses).
 *
 *   kmean[s][b][c] = (sum over t in [b*B, min(b*B+B, len_s)) of
 *                     idx_k[s][t][c]) / (number of those t)
 *
 * summed in fp32 in a fixed order (so the result is deterministic but, unlike
 * the max, carries rounding: within (n+1) * 2^-24 * sum|x| / n of the exact
 * mean for a block of n tokens).  Arguments as msa_index_pool, except that
 * only the range form (blk_begin >= 0) and the last-block form
 * (blk_begin == -1) exist; blk_begin == -2 returns MSA_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------ */
int msa_index_pool_mean(const float *idx_k, int32_t n_seq, int64_t len_max,
                        const int64_t *seq_len, int32_t d_idx, int32_t block,
                        int64_t blk_begin, int64_t blk_end, float *kmean,
                        int64_t nb_max, void *stream);

/* --------------------------------------------------------------------------
 * msa_index_topk -- prefill scores and causal top-K for one sequence.
 * [YLY] "索引分支（Index Branch）"; [CXT] section 3.3 "Prefilling 与 Decoding
 * 的差异化优化" (prefill scores every block for every query).
 *
 * Query i sits at position p = q_pos0 + i, own = p / B.  Its candidates are
 * the blocks b < own, scored in fp32 by s[b] = sum_c idx_q[i][c]*kmax[b][c]
 * (fp32 products and sums in an unspecified order, so scores within the fp32
 * dot-product error bound of each other may rank either way); it keeps the
 * best min(K-1, own) by (score desc, block asc), adds own, and writes them
 * ascending to sel[i][0..], padding with -1 up to K.
 *
 *   idx_q  [n_q][d_idx] fp32;  kmax [nb][d_idx] fp32 with
 *          nb >= own of the last query + 1
 *   sel    [n_q][K] int32 (output)
 * ------------------------------------------------------------------------ */
int msa_index_topk(const float *idx_q, int64_t n_q, int64_t q_pos0,
                   const float *kmax, int64_t nb, int32_t d_idx, int32_t block,
                   int32_t topk, int32_t *sel, void *stream);

/* --------------------------------------------------------------------------
 * msa_index_topk_window -- the same selection with a forced local window of
 * `window` blocks, after [CXT] section 3.3's sketch, which always keeps the
 * blocks nearest the query besides the top-scored ones.  For query p with
 * own = p / B the blocks max(0, own-window+1) .. own are forced; the
 * candidates are the blocks below them, of which the best K - window are kept
 * by (score desc, block asc).  The row is ascending and -1 padded as before;
 * window = 1 is msa_index_topk.  Requires 1 <= window <= K
 * (else MSA_ERR_INVALID_ARG).
 * ------------------------------------------------------------------------ */
int msa_index_topk_window(const float *idx_q, int64_t n_q, int64_t q_pos0,
                          const float *kmax, int64_t nb, int32_t d_idx, int32_t block,
                          int32_t topk, int32_t window, int32_t *sel, void *stream);

/* --------------------------------------------------------------------------
 * msa_index_topk_decode -- the same selection for one new query per
 * sequence ([CXT] section 3.3: decode scores only the new token).  Sequence
 * s's query sits at position seq_len[s] - 1 (its index key already pooled).
 *
 *   idx_q    [n_seq][d_idx] fp32
 *   seq_len  device int64 [n_seq], 1 <= len_s <= nb_max * B
 *   kmax     [n_seq][nb_max][d_idx] fp32
 *   sel      [n_seq][K] int32 (output)
 *   ws       device scratch of msa_topk_decode_workspace_bytes() bytes
 * ------------------------------------------------------------------------ */
size_t msa_topk_decode_workspace_bytes(int32_t n_seq, int64_t nb_max,
                                       int32_t topk);
int msa_index_topk_decode(const float *idx_q, int32_t n_seq,
                          const int64_t *seq_len, const float *kmax,
                          int64_t nb_max, int32_t d_idx, int32_t block,
                          int32_t topk, int32_t *sel, void *ws,
                          size_t ws_bytes, void *stream);
/* The decode selection with the local window of msa_index_topk_window
 * (window = 1 is msa_index_topk_decode); same workspace. */
int msa_index_topk_decode_window(const float *idx_q, int32_t n_seq,
                                 const int64_t *seq_len, const float *kmax,
                                 int64_t nb_max, int32_t d_idx, int32_t block,
                                 int32_t topk, int32_t window, int32_t *sel, void *ws,
                                 size_t ws_bytes, void *stream);

/* --------------------------------------------------------------------------
 * msa_index_topk_batch -- the same selection for a batch of queries drawn
 * from several sequences, each at its own position ([CXT] section 3.3: the
 * index branch scores a query against the block summaries of its own
 * sequence; [YLY] "索引分支（Index Branch）").  Query i belongs to sequence
 * q_seq[i] and sits at position p = q_pos[i], own = p / B; its row is that of
 * msa_index_topk for that query against sequence q_seq[i]'s summaries.  A
 * query with q_seq[i] outside [0, n_seq) or p outside [0, nb_max * B) gets a
 * row of -1 (no error: the arrays are on the device).
 *
 *   idx_q  [n_q][d_idx] fp32
 *   q_seq  device int32 [n_q];  q_pos device int64 [n_q]
 *   kmax   [n_seq][nb_max][d_idx] fp32 (rows past a sequence's own block of
 *          the query are read but never selected)
 *   sel    [n_q][K] int32 (output)
 *   ws     device scratch of msa_topk_batch_workspace_bytes() bytes
 *
 * n_q = 0 returns MSA_OK and launches nothing; 1 <= n_seq <= 65535 and
 * nb_max <= 65535 * 64 (else MSA_ERR_INVALID_ARG).
 * ------------------------------------------------------------------------ */
size_t msa_topk_batch_workspace_bytes(int64_t n_q, int64_t nb_max, int32_t topk);
int msa_index_topk_batch(const float *idx_q, int64_t n_q, const int32_t *q_seq,
                         const int64_t *q_pos, const float *kmax, int32_t n_seq,
                         int64_t nb_max, int32_t d_idx, int32_t block, int32_t topk,
                         int32_t *sel, void *ws, size_t ws_bytes, void *stream);

/* --------------------------------------------------------------------------
 * msa_invert_selection -- the queries that hit each KV block, as CSR.
 * [CXT] section 2.2: the KV-outer loop needs, per block, the queries that
 * chose it.  Histogram, prefix sum and a deterministic scatter:
 *
 *   row_ptr[b+1] - row_ptr[b] = |{i : b in sel[i]}|,  row_ptr[0] = 0
 *   q_list[row_ptr[b] ..]     = those i, ascending
 *   slot[i][k]                = position of (i, sel[i][k]) in q_list,
 *                               -1 where sel[i][k] == -1
 *
 *   sel      [n_q][K] int32, entries -1 or in [0, n_blocks), no repeats in a row
 *   row_ptr  [n_blocks+1] int32;  q_list [n_q*K] int32 (capacity);
 *   slot     [n_q][K] int32 (outputs); n_q * K < 2^31
 *   ws       device scratch of msa_invert_workspace_bytes() bytes
 * ------------------------------------------------------------------------ */
size_t msa_invert_workspace_bytes(int64_t n_q, int32_t topk, int64_t n_blocks);
int msa_invert_selection(const int32_t *sel, int64_t n_q, int32_t topk,
                         int64_t n_blocks, int32_t *row_ptr, int32_t *q_list,
                         int32_t *slot, void *ws, size_t ws_bytes,
                         void *stream);

/* --------------------------------------------------------------------------
 * msa_sparse_gqa_prefill -- GQA over each query's selected blocks, KV outer.
 * [YLY] "稀疏分支（Sparse Branch）"; [CXT] sections 2.2 and 2.3.
 *
 * Query i (position p = q_pos0 + i), head h, KV head g = h / (Hq/Hkv):
 *   keys  = union over b in sel[i] of {t : b*B <= t <= min(b*B+B-1, p)}
 *   o     = softmax(scale * q.k_t) . v_t over those keys,
 *   lse   = natural log of sum_t exp(scale * q.k_t).
 * Each (block, KV head) pair is streamed once per group of queries that chose
 * it; every non-own block yields a partial (o, lse) per (query, head) in the
 * workspace, and the own-block pass merges them by log-sum-exp.
 *
 *   q     [n_q][Hq][d]            dtype (fp32 or bf16 bits)
 *   k, v  [Hkv][kv_stride][d]     dtype; q_pos0 + n_q <= kv_stride
 *   sel   [n_q][K] from msa_index_topk with the same q_pos0 and B;
 *         row_ptr, q_list, slot from msa_invert_selection(sel, n_q, K,
 *         ceil((q_pos0+n_q)/B)).  Results are undefined for other inputs
 *         (out-of-range entries are skipped, never dereferenced).
 *   o     [n_q][Hq][d] fp32;  lse [n_q][Hq] fp32 (may be NULL)
 *   ws    device scratch of msa_prefill_workspace_bytes(dtype, ...) bytes; it
 *         holds one partial record per (non-own pair, query head): fp32 for
 *         fp32 inputs; for bf16 with d = 128 the output as fp16 scaled by a
 *         power of two (values below 1; relative precision 2^-11 of the
 *         record's max |o|) plus its fp32 log-sum-exp and exponent
 *   Supported: fp32 and bf16 with d in {64, 128}, d = 256 with Hq/Hkv <= 4;
 *   Hq/Hkv in {1, 2, 4, 8, 16}.
 * ------------------------------------------------------------------------ */
size_t msa_prefill_workspace_bytes(int32_t dtype, int64_t q_pos0, int64_t n_q,
                                   int32_t hq, int32_t d, int32_t block,
                                   int32_t topk);
int msa_sparse_gqa_prefill(const void *q, const void *k, const void *v,
                           int32_t dtype, int64_t kv_stride, int64_t q_pos0,
                           int64_t n_q, int32_t hq, int32_t hkv, int32_t d,
                           int32_t block, const int32_t *sel, int32_t topk,
                           const int32_t *row_ptr, const int32_t *q_list,
                           const int32_t *slot, float scale, float *o,
                           float *lse, void *ws, size_t ws_bytes,
                           void *stream);

/* --------------------------------------------------------------------------
 * msa_sparse_gqa_prefill_paged -- msa_sparse_gqa_prefill for a chunk of
 * queries against a paged bf16 KV cache ([CXT] section 3.3: prefill of a
 * request's next chunk against the cache already built, the cache kept in
 * block-granular pages, section 3.2).  Same page layout as
 * msa_sparse_gqa_decode_paged: a page holds one MSA block of every KV head,
 *
 *   k_pages, v_pages  [n_pages][Hkv][B][d] bf16
 *   block_table       [max_blocks] int32: block b of the sequence (keys
 *                     b*B .. b*B+B-1) lives in page block_table[b];
 *                     ceil((q_pos0 + n_q) / B) <= max_blocks
 *   q, sel, row_ptr, q_list, slot, o, lse, scale, ws as msa_sparse_gqa_prefill
 *                     (ws: msa_prefill_workspace_bytes with dtype MSA_BF16)
 * Only the table entries of blocks the selection uses are read.  An entry
 * outside [0, n_pages) is clamped into the pool (nothing outside it is
 * read); the outputs of the queries that use such a block are unspecified.
 * Results are bit-identical to msa_sparse_gqa_prefill on the same keys and
 * values laid out contiguously.
 * Supported: bf16, d = 128, Hq/Hkv in {1, 2, 4, 8, 16}.
 * ------------------------------------------------------------------------ */
int msa_sparse_gqa_prefill_paged(const void *q, const void *k_pages, const void *v_pages,
                                 int64_t n_pages, const int32_t *block_table,
                                 int32_t max_blocks, int64_t q_pos0, int64_t n_q, int32_t hq,
                                 int32_t hkv, int32_t d, int32_t block, const int32_t *sel,
                                 int32_t topk, const int32_t *row_ptr, const int32_t *q_list,
                                 const int32_t *slot, float scale, float *o, float *lse,
                                 void *ws, size_t ws_bytes, void *stream);

/* --------------------------------------------------------------------------
 * msa_prefill_varlen -- the whole prefill path (pool, top-K, CSR, sparse
 * GQA with merge) for several sequences in one call, each a chunk of queries
 * against its own cache ([CXT] section 3.3: prefill over a batch of
 * requests of different lengths; the queries of a chunk attend to the
 * blocks already in the cache).  Packed layouts with host offsets:
 *
 *   cu_q, cu_kv  HOST int64 [n_seq+1], cu_q[0] = cu_kv[0] = 0, nondecreasing;
 *                sequence s has qn = cu_q[s+1]-cu_q[s] queries and
 *                kvn = cu_kv[s+1]-cu_kv[s] >= qn cached tokens, its queries
 *                being the last qn tokens (positions kvn-qn .. kvn-1)
 *   q            [cu_q[n]][Hq][d] dtype;  idx_q [cu_q[n]][d_idx] fp32
 *   k, v         [Hkv][cu_kv[n]][d] dtype;  idx_k [cu_kv[n]][d_idx] fp32
 *   sel          [cu_q[n]][K] int32 out (each sequence's own block indices)
 *   o, lse       [cu_q[n]][Hq][d], [cu_q[n]][Hq] fp32 out (lse may be NULL)
 *   ws           device scratch of msa_prefill_varlen_workspace_bytes()
 * bf16 with d = 128: the sequences run in chains of up to 64 consecutive
 * sequences (fewer when the chain's workspace would pass 16 GiB; a single
 * larger sequence is a chain of its own), each chain one launch sequence
 * over all of its sequences (the blocks of all of them numbered in one CSR),
 * so many short requests fill the GPU together.  Other types and head sizes:
 * one sequence after another with the single-sequence kernels.  Everything is
 * enqueued on `stream`; nothing is synchronised.  The workspace holds the
 * largest chain's (or sequence's) summaries, CSR and partial records, so a
 * long sequence is best split by the caller into query chunks.  Results are
 * bit-identical to the single-sequence entry points on each sequence.
 * Supported as msa_sparse_gqa_prefill.
 * ------------------------------------------------------------------------ */
size_t msa_prefill_varlen_workspace_bytes(int32_t dtype, int32_t n_seq, const int64_t *cu_q,
                                          const int64_t *cu_kv, int32_t hq, int32_t d,
                                          int32_t d_idx, int32_t block, int32_t topk);
int msa_prefill_varlen(const void *q, const void *k, const void *v, const float *idx_q,
                       const float *idx_k, int32_t dtype, int32_t n_seq, const int64_t *cu_q,
                       const int64_t *cu_kv, int32_t hq, int32_t hkv, int32_t d,
                       int32_t d_idx, int32_t block, int32_t topk, float scale, int32_t *sel,
                       float *o, float *lse, void *ws, size_t ws_bytes, void *stream);

/* --------------------------------------------------------------------------
 * msa_sparse_gqa_decode -- one new query per sequence over its selected
 * blocks ([CXT] section 3.3, decode), split over (block, key chunk) and
 * merged by log-sum-exp.  Sequence s's query sits at position seq_len[s]-1;
 * its own key and value are already in the cache.
 *
 *   q        [n_seq][Hq][d] dtype
 *   k_cache, v_cache  [n_seq][Hkv][len_max][d] dtype
 *   seq_len  device int64 [n_seq], 1 <= len_s <= len_max
 *   sel      [n_seq][K] int32 from msa_index_topk_decode
 *   o        [n_seq][Hq][d] fp32;  lse [n_seq][Hq] fp32 (may be NULL)
 *   ws       device scratch of msa_decode_workspace_bytes() bytes
 *   Supported: fp32 and bf16 with d in {64, 128}, bf16 with d = 256;
 *   Hq/Hkv in {1, 2, 4, 8, 16}.  n_seq * Hkv * K <= 2^28 (else
 *   MSA_ERR_INVALID_ARG).
 * ------------------------------------------------------------------------ */
size_t msa_decode_workspace_bytes(int32_t n_seq, int32_t hq, int32_t d,
                                  int32_t block, int32_t topk);
int msa_sparse_gqa_decode(const void *q, const void *k_cache,
                          const void *v_cache, int32_t dtype, int32_t n_seq,
                          int64_t len_max, const int64_t *seq_len, int32_t hq,
                          int32_t hkv, int32_t d, int32_t block,
                          const int32_t *sel, int32_t topk, float scale,
                          float *o, float *lse, void *ws, size_t ws_bytes,
                          void *stream);

/* --------------------------------------------------------------------------
 * msa_sparse_gqa_decode_paged -- msa_sparse_gqa_decode over a paged KV cache,
 * with bf16 or FP8 keys and values ([CXT] section 3.3's KV cache management:
 * block-granular allocation, and KV kept in reduced precision).  A page holds
 * one MSA block of one KV head:
 *
 *   k_pages, v_pages  [n_pages][Hkv][B][d], kv_dtype MSA_BF16 or MSA_FP8_E4M3
 *   k_scale, v_scale  [n_pages][Hkv] fp32 (FP8 only; ignored for bf16):
 *                     key row = k_scale[page][g] * e4m3 value, likewise v
 *   block_table       [n_seq][max_blocks] int32: logical block b of sequence
 *                     s (keys b*B .. b*B+B-1) lives in page block_table[s][b]
 *   q                 [n_seq][Hq][d] bf16; seq_len, sel, o, lse, ws, scale as
 *                     msa_sparse_gqa_decode (ws: msa_decode_workspace_bytes),
 *                     with len_s <= max_blocks * B
 * Only the table entries of selected blocks are read; an entry outside
 * [0, n_pages) makes that block count as attending no keys (nothing outside
 * the pool is read).  Dequantisation is exact up to fp32 rounding of the
 * scaled scores and outputs (e4m3 values are exact in bf16).
 * Supported: d = 128, Hq/Hkv in {1, 2, 4, 8, 16}; n_seq * Hkv * K <= 2^28.
 * ------------------------------------------------------------------------ */
int msa_sparse_gqa_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                                int32_t kv_dtype, const float *k_scale,
                                const float *v_scale, int64_t n_pages,
                                const int32_t *block_table, int32_t max_blocks,
                                int32_t n_seq, const int64_t *seq_len, int32_t hq,
                                int32_t hkv, int32_t d, int32_t block,
                                const int32_t *sel, int32_t topk, float scale, float *o,
                                float *lse, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * msa_decode_step -- one generation step of the whole path, fused
 * [CXT 3.3: the new token is appended, its block summary updated, the query
 * scored against the summaries, the top-K blocks attended]:
 *   1. append the new token at position L = seq_len[s] of every sequence:
 *      k_cache[s][g][L] = k_new[s][g], v_cache likewise, and
 *      idx_k_cache[s][L] = idx_k_new[s] when idx_k_cache is not NULL;
 *   2. running block max: kmax[s][L/B] = idx_k_new[s] when L % B == 0 (the
 *      token opens a block), else the elementwise max of the two (exact, with
 *      -0 below +0, as msa_index_pool);
 *   3. the query at position L scores every earlier block summary and keeps
 *      the causal top-K with its own block L/B forced (msa_index_topk_decode's
 *      rule); the row is written to sel;
 *   4. sparse GQA over the selected blocks, keys 0..L (msa_sparse_gqa_decode).
 * seq_len is read, not advanced: the caller adds one per step.  All of it is
 * enqueued on `stream` as three kernels, with no allocation and no host
 * synchronisation, so a step can be captured in a HIP graph.
 *   q          [n_seq][Hq][d] bf16, the new token's queries
 *   k_new/v_new [n_seq][Hkv][d] bf16;  idx_q, idx_k_new [n_seq][d_idx] fp32
 *   k_cache/v_cache [n_seq][Hkv][len_max][d] bf16 (written at L)
 *   idx_k_cache [n_seq][len_max][d_idx] fp32 or NULL;  kmax [n_seq][nb_max][d_idx]
 *   Requires L < len_max and L / B < nb_max for every sequence; a sequence
 *   without room gets no append and unspecified outputs (nothing outside the
 *   given buffers is written).
 *   sel [n_seq][K] int32 out;  o [n_seq][Hq][d] fp32;  lse [n_seq][Hq] (may be NULL)
 *   ws  device scratch of msa_decode_step_workspace_bytes() bytes
 *   Supported: bf16, d = 128, Hq/Hkv in {1, 2, 4, 8, 16}.
 *   n_seq * Hkv * K <= 2^28 (else MSA_ERR_INVALID_ARG).
 * ------------------------------------------------------------------------ */
size_t msa_decode_step_workspace_bytes(int32_t n_seq, int64_t nb_max, int32_t hq,
                                       int32_t d, int32_t block, int32_t topk);
int msa_decode_step(const void *q, const void *k_new, const void *v_new,
                    const float *idx_q, const float *idx_k_new, void *k_cache,
                    void *v_cache, float *idx_k_cache, float *kmax, int32_t dtype,
                    int32_t n_seq, int64_t len_max, int64_t nb_max,
                    const int64_t *seq_len, int32_t hq, int32_t hkv, int32_t d,
                    int32_t d_idx, int32_t block, int32_t topk, float scale,
                    int32_t *sel, float *o, float *lse, void *ws, size_t ws_bytes,
                    void *stream);

/* --------------------------------------------------------------------------
 * msa_decode_step_paged -- msa_decode_step with the keys and values in a
 * paged bf16 cache ([CXT] section 3.3: block-granular KV cache management,
 * the new token appended into its block's page).  Page layout and table as
 * msa_sparse_gqa_decode_paged:
 *
 *   k_pages, v_pages  [n_pages][Hkv][B][d] bf16; the new token's K and V
 *                     rows are written at row L % B of page block_table[s][L / B]
 *   block_table       [n_seq][max_blocks] int32 (the caller places a page
 *                     there before the step whose token opens the block)
 *   idx_k_cache       [n_seq][len_max][d_idx] fp32 or NULL; len_max bounds L
 *   everything else as msa_decode_step (ws: msa_decode_step_workspace_bytes)
 * Requires L < len_max, L / B < nb_max and L / B < max_blocks with a table
 * entry in [0, n_pages) for the new token's block; a sequence without them
 * gets no append and unspecified outputs (nothing outside the given buffers
 * is written).  A selected block whose entry is outside [0, n_pages) attends
 * no keys.  Results are bit-identical to msa_decode_step on the same cache
 * laid out contiguously.
 * Supported: d = 128, Hq/Hkv in {1, 2, 4, 8, 16}; n_seq * Hkv * K <= 2^28.
 * ------------------------------------------------------------------------ */
int msa_decode_step_paged(const void *q, const void *k_new, const void *v_new,
                          const float *idx_q, const float *idx_k_new, void *k_pages,
                          void *v_pages, int64_t n_pages, const int32_t *block_table,
                          int32_t max_blocks, float *idx_k_cache, float *kmax, int32_t n_seq,
                          int64_t len_max, int64_t nb_max, const int64_t *seq_len, int32_t hq,
                          int32_t hkv, int32_t d, int32_t d_idx, int32_t block, int32_t topk,
                          float scale, int32_t *sel, float *o, float *lse, void *ws,
                          size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * msa_decode_step_noalloc -- msa_decode_step for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Arguments and
 * results are those of msa_decode_step without ws / ws_bytes; the scratch it
 * needs (msa_decode_step_workspace_bytes() of the same shape) comes from a
 * static device array of msa_decode_step_noalloc_max_bytes() bytes (32 MiB)
 * that the library holds on each device it runs on until the process ends.
 * Nothing is allocated.  A shape whose scratch exceeds the maximum returns
 * MSA_ERR_WORKSPACE (for example dec16's 16 sequences x 8 KV heads need
 * about 17 MiB; about 500 such sequences at block 512, top-K 8 would not
 * fit).  Every call on one device shares that device's array: calls that
 * overlap on one device (different streams, different host threads without
 * ordering) race and give undefined results; calls ordered on one stream are
 * safe.  The first call on a device looks up the array's address (once).
 * ------------------------------------------------------------------------ */
size_t msa_decode_step_noalloc_max_bytes(void);
int msa_decode_step_noalloc(const void *q, const void *k_new, const void *v_new,
                            const float *idx_q, const float *idx_k_new, void *k_cache,
                            void *v_cache, float *idx_k_cache, float *kmax, int32_t dtype,
                            int32_t n_seq, int64_t len_max, int64_t nb_max,
                            const int64_t *seq_len, int32_t hq, int32_t hkv, int32_t d,
                            int32_t d_idx, int32_t block, int32_t topk, float scale,
                            int32_t *sel, float *o, float *lse, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H */
