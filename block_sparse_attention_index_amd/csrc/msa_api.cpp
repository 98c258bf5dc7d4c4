// msa_api.cpp -- the C-ABI entry points declared in include/msa.h: argument
// validation, workspace sizing and kernel selection.  Every check runs before
// anything is enqueued, so an error leaves the outputs untouched.  Nothing
// here allocates device memory, and nothing falls back to another path: an
// unsupported shape is reported as MSA_ERR_UNSUPPORTED.
#include "msa.h"

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "msa_internal.h"

namespace {

constexpr int32_t kMaxBlock = 4096;
constexpr int32_t kMaxTopk = 64;
constexpr int64_t kMaxGridY = 65535;
// (sequence, KV head, selected block) work items of one decode call: the
// streaming kernel numbers their segments in 32 bits
constexpr int64_t kMaxDecodeItems = int64_t(1) << 28;
// Shape limits that keep every byte count below 2^60 (they are computed in
// 64-bit arithmetic): token positions and counts, heads, head size.
constexpr int64_t kMaxTokens = int64_t(1) << 40;
constexpr int64_t kMaxHeads = int64_t(1) << 16;
constexpr int32_t kMaxD = 1024;
bool bytes_fit(__int128 x) { return x >= 0 && x < ((__int128)1 << 60); }
// n_q * topk < 2^31 - 1 (query-block pairs are numbered in 32 bits), without
// forming the product
bool pairs_ok(int64_t n_q, int32_t topk) {
  return n_q >= 0 && topk >= 1 && n_q <= (int64_t)(INT32_MAX - 1) / topk;
}
// Partial records of a prefill call: at most (q_pos0 + n_q) * (K - 1) pairs,
// each Hq * (d + 2) floats, plus per-block tables.
bool prefill_shape_ok(int64_t q_pos0, int64_t n_q, int32_t hq, int32_t d, int32_t block,
                      int32_t topk) {
  if (q_pos0 < 0 || n_q < 0 || q_pos0 > kMaxTokens || n_q > kMaxTokens || hq < 1 ||
      hq > kMaxHeads || d < 1 || d > kMaxD)
    return false;
  const __int128 toks = (__int128)q_pos0 + n_q;
  // blocks, tiles and CSR offsets are numbered in 32 bits
  if (toks / block >= INT32_MAX / 2) return false;
  return bytes_fit(toks * topk * hq * (d + 2) * 4 + (toks / block + 1) * 4096);
}
// Decode partials: one record of Hq * (d + 1) floats per (sequence, selected
// block, 128-key segment), plus the scan's candidate lists.
bool decode_shape_ok(int32_t n_seq, int64_t nb_max, int32_t hq, int32_t d, int32_t block,
                     int32_t topk) {
  if (n_seq < 1 || n_seq > kMaxGridY || nb_max < 1 || nb_max > INT32_MAX || hq < 1 ||
      hq > kMaxHeads || d < 1 || d > kMaxD)
    return false;
  return bytes_fit((__int128)n_seq * hq * topk * ((block + 127) / 128) * (d + 1) * 4 +
                   (__int128)n_seq * (nb_max / 64 + 1) * topk * 8);
}

bool block_ok(int32_t b) { return b >= 16 && b <= kMaxBlock && b % 16 == 0; }
bool topk_ok(int32_t k) { return k >= 1 && k <= kMaxTopk; }
bool didx_ok(int32_t d) {
  return d >= 1 && d <= 1024 && (d % 4 == 0 || d <= 256);
}
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int status_of(hipError_t e) { return e == hipSuccess ? MSA_OK : MSA_ERR_HIP; }
hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

}  // namespace

namespace msa {
bool generic_prefill_supported(int32_t d, int32_t group);
hipError_t launch_prefill_generic(const void *q, const void *k, const void *v,
                                  int32_t dtype, int64_t kv_stride,
                                  int64_t q_pos0, int64_t n_q, int32_t hq,
                                  int32_t hkv, int32_t d, int32_t block,
                                  const int32_t *sel, int32_t topk,
                                  const int32_t *row_ptr,
                                  const int32_t *q_list, const int32_t *slot,
                                  float scale, float *o, float *lse, void *ws,
                                  hipStream_t st);

bool mfma_prefill_supported(int32_t dtype, int32_t d, int32_t group);
hipError_t launch_prefill_mfma(const void *q, const void *k, const void *v,
                               int64_t kv_stride, int64_t q_pos0, int64_t n_q,
                               int32_t hq, int32_t hkv, int32_t d,
                               int32_t block, const int32_t *sel, int32_t topk,
                               const int32_t *row_ptr, const int32_t *q_list,
                               const int32_t *slot, float scale, float *o,
                               float *lse, void *ws, hipStream_t st);

bool prefill_supported(int32_t dtype, int32_t d, int32_t group) {
  if (dtype != MSA_F32 && dtype != MSA_BF16) return false;
  return mfma_prefill_supported(dtype, d, group) ||
         generic_prefill_supported(d, group);
}

hipError_t launch_prefill(const void *q, const void *k, const void *v,
                          int32_t dtype, int64_t kv_stride, int64_t q_pos0,
                          int64_t n_q, int32_t hq, int32_t hkv, int32_t d,
                          int32_t block, const int32_t *sel, int32_t topk,
                          const int32_t *row_ptr, const int32_t *q_list,
                          const int32_t *slot, float scale, float *o,
                          float *lse, void *ws, hipStream_t st) {
  // bf16 with d = 128 runs on the matrix cores; everything else (fp32
  // inputs, other head sizes) on the fp32 VALU kernels.
  if (mfma_prefill_supported(dtype, d, hq / hkv))
    return launch_prefill_mfma(q, k, v, kv_stride, q_pos0, n_q, hq, hkv, d,
                               block, sel, topk, row_ptr, q_list, slot, scale,
                               o, lse, ws, st);
  return launch_prefill_generic(q, k, v, dtype, kv_stride, q_pos0, n_q, hq, hkv,
                                d, block, sel, topk, row_ptr, q_list, slot,
                                scale, o, lse, ws, st);
}
}  // namespace msa

extern "C" {

const char *msa_status_string(int status) {
  switch (status) {
    case MSA_OK:
      return "MSA_OK";
    case MSA_ERR_INVALID_ARG:
      return "MSA_ERR_INVALID_ARG: invalid argument";
    case MSA_ERR_UNSUPPORTED:
      return "MSA_ERR_UNSUPPORTED: no kernel for this configuration";
    case MSA_ERR_WORKSPACE:
      return "MSA_ERR_WORKSPACE: workspace too small";
    case MSA_ERR_HIP:
      return "MSA_ERR_HIP: HIP launch or runtime error";
    default:
      return "unknown msa status";
  }
}

int msa_index_pool(const float *idx_k, int32_t n_seq, int64_t len_max,
                   const int64_t *seq_len, int32_t d_idx, int32_t block,
                   int64_t blk_begin, int64_t blk_end, float *kmax,
                   int64_t nb_max, void *stream) {
  if (!idx_k || !kmax || n_seq < 1 || n_seq > kMaxGridY || len_max < 1 ||
      !didx_ok(d_idx) || !block_ok(block) || nb_max < cdiv(len_max, block))
    return MSA_ERR_INVALID_ARG;
  if (blk_begin < -2 || (blk_begin >= 0 && (blk_end <= blk_begin || blk_end > nb_max ||
                                             blk_end - blk_begin > INT32_MAX)))
    return MSA_ERR_INVALID_ARG;
  return status_of(msa::launch_pool(idx_k, n_seq, len_max, seq_len, d_idx,
                                    block, blk_begin, blk_end, kmax, nb_max,
                                    as_stream(stream)));
}

int msa_index_pool_mean(const float *idx_k, int32_t n_seq, int64_t len_max,
                        const int64_t *seq_len, int32_t d_idx, int32_t block,
                        int64_t blk_begin, int64_t blk_end, float *kmean,
                        int64_t nb_max, void *stream) {
  if (!idx_k || !kmean || n_seq < 1 || n_seq > kMaxGridY || len_max < 1 ||
      !didx_ok(d_idx) || !block_ok(block) || nb_max < cdiv(len_max, block))
    return MSA_ERR_INVALID_ARG;
  if (blk_begin < -1 || (blk_begin >= 0 && (blk_end <= blk_begin || blk_end > nb_max ||
                                             blk_end - blk_begin > INT32_MAX)))
    return MSA_ERR_INVALID_ARG;
  return status_of(msa::launch_pool_mean(idx_k, n_seq, len_max, seq_len, d_idx,
                                         block, blk_begin, blk_end, kmean, nb_max,
                                         as_stream(stream)));
}

int msa_index_topk_window(const float *idx_q, int64_t n_q, int64_t q_pos0,
                          const float *kmax, int64_t nb, int32_t d_idx, int32_t block,
                          int32_t topk, int32_t window, int32_t *sel, void *stream) {
  if (!idx_q || !kmax || !sel || n_q < 0 || q_pos0 < 0 || !didx_ok(d_idx) ||
      !block_ok(block) || !topk_ok(topk) || nb < 1 || window < 1 || window > topk)
    return MSA_ERR_INVALID_ARG;
  if (n_q == 0) return MSA_OK;
  if ((q_pos0 + n_q - 1) / block >= nb || (q_pos0 + n_q - 1) / block > INT32_MAX)
    return MSA_ERR_INVALID_ARG;
  return status_of(msa::launch_topk_prefill(idx_q, n_q, q_pos0, kmax, nb, d_idx,
                                            block, topk, window, sel,
                                            as_stream(stream)));
}

int msa_index_topk(const float *idx_q, int64_t n_q, int64_t q_pos0,
                   const float *kmax, int64_t nb, int32_t d_idx, int32_t block,
                   int32_t topk, int32_t *sel, void *stream) {
  return msa_index_topk_window(idx_q, n_q, q_pos0, kmax, nb, d_idx, block, topk, 1, sel,
                               stream);
}

size_t msa_topk_decode_workspace_bytes(int32_t n_seq, int64_t nb_max,
                                       int32_t topk) {
  if (n_seq < 1 || n_seq > kMaxGridY || nb_max < 1 || nb_max > INT32_MAX || !topk_ok(topk))
    return 0;
  return msa::topk_decode_ws_bytes(n_seq, nb_max, topk);
}

int msa_index_topk_decode_window(const float *idx_q, int32_t n_seq,
                                 const int64_t *seq_len, const float *kmax,
                                 int64_t nb_max, int32_t d_idx, int32_t block,
                                 int32_t topk, int32_t window, int32_t *sel, void *ws,
                                 size_t ws_bytes, void *stream) {
  if (!idx_q || !seq_len || !kmax || !sel || !ws || n_seq < 1 ||
      n_seq > kMaxGridY || nb_max < 1 || nb_max > INT32_MAX ||
      !didx_ok(d_idx) || !block_ok(block) || !topk_ok(topk) || window < 1 ||
      window > topk)
    return MSA_ERR_INVALID_ARG;
  if (ws_bytes < msa::topk_decode_ws_bytes(n_seq, nb_max, topk))
    return MSA_ERR_WORKSPACE;
  return status_of(msa::launch_topk_decode(idx_q, n_seq, seq_len, kmax, nb_max,
                                           d_idx, block, topk, window, sel, ws,
                                           as_stream(stream)));
}

// One workgroup per (query, 64-block chunk): the chunks run along grid y.
static bool batch_dims_ok(int64_t n_q, int64_t nb_max) {
  return n_q >= 0 && n_q <= INT32_MAX && nb_max >= 1 &&
         (nb_max + 63) / 64 <= kMaxGridY;
}

size_t msa_topk_batch_workspace_bytes(int64_t n_q, int64_t nb_max, int32_t topk) {
  if (!batch_dims_ok(n_q, nb_max) || !topk_ok(topk)) return 0;
  return msa::topk_batch_ws_bytes(n_q, nb_max, topk);
}

int msa_index_topk_batch(const float *idx_q, int64_t n_q, const int32_t *q_seq,
                         const int64_t *q_pos, const float *kmax, int32_t n_seq,
                         int64_t nb_max, int32_t d_idx, int32_t block, int32_t topk,
                         int32_t *sel, void *ws, size_t ws_bytes, void *stream) {
  if (!batch_dims_ok(n_q, nb_max) || n_seq < 1 || n_seq > kMaxGridY ||
      !didx_ok(d_idx) || !block_ok(block) || !topk_ok(topk))
    return MSA_ERR_INVALID_ARG;
  if (n_q == 0) return MSA_OK;
  if (!idx_q || !q_seq || !q_pos || !kmax || !sel || !ws) return MSA_ERR_INVALID_ARG;
  if (ws_bytes < msa::topk_batch_ws_bytes(n_q, nb_max, topk)) return MSA_ERR_WORKSPACE;
  return status_of(msa::launch_topk_batch(idx_q, n_q, q_seq, q_pos, kmax, n_seq, nb_max,
                                          d_idx, block, topk, sel, ws, as_stream(stream)));
}

int msa_index_topk_decode(const float *idx_q, int32_t n_seq,
                          const int64_t *seq_len, const float *kmax,
                          int64_t nb_max, int32_t d_idx, int32_t block,
                          int32_t topk, int32_t *sel, void *ws,
                          size_t ws_bytes, void *stream) {
  return msa_index_topk_decode_window(idx_q, n_seq, seq_len, kmax, nb_max, d_idx, block,
                                      topk, 1, sel, ws, ws_bytes, stream);
}

size_t msa_invert_workspace_bytes(int64_t n_q, int32_t topk, int64_t n_blocks) {
  if (!topk_ok(topk) || !pairs_ok(n_q, topk) || n_blocks < 1 || n_blocks >= INT32_MAX)
    return 0;
  return msa::invert_ws_bytes(n_q, topk, n_blocks);
}

int msa_invert_selection(const int32_t *sel, int64_t n_q, int32_t topk,
                         int64_t n_blocks, int32_t *row_ptr, int32_t *q_list,
                         int32_t *slot, void *ws, size_t ws_bytes,
                         void *stream) {
  if (!sel || !row_ptr || !q_list || !slot || !ws || !topk_ok(topk) ||
      !pairs_ok(n_q, topk) || n_blocks < 1 || n_blocks >= INT32_MAX)
    return MSA_ERR_INVALID_ARG;
  if (ws_bytes < msa::invert_ws_bytes(n_q, topk, n_blocks))
    return MSA_ERR_WORKSPACE;
  return status_of(msa::launch_invert(sel, n_q, topk, n_blocks, row_ptr, q_list,
                                      slot, ws, as_stream(stream)));
}

size_t msa_prefill_workspace_bytes(int32_t dtype, int64_t q_pos0, int64_t n_q,
                                   int32_t hq, int32_t d, int32_t block,
                                   int32_t topk) {
  if ((dtype != MSA_F32 && dtype != MSA_BF16) || !block_ok(block) || !topk_ok(topk) ||
      !prefill_shape_ok(q_pos0, n_q, hq, d, block, topk))
    return 0;
  return msa::prefill_ws_bytes(dtype, q_pos0, n_q, hq, d, block, topk);
}

int msa_sparse_gqa_prefill(const void *q, const void *k, const void *v,
                           int32_t dtype, int64_t kv_stride, int64_t q_pos0,
                           int64_t n_q, int32_t hq, int32_t hkv, int32_t d,
                           int32_t block, const int32_t *sel, int32_t topk,
                           const int32_t *row_ptr, const int32_t *q_list,
                           const int32_t *slot, float scale, float *o,
                           float *lse, void *ws, size_t ws_bytes,
                           void *stream) {
  if (!q || !k || !v || !sel || !row_ptr || !q_list || !slot || !o || !ws ||
      (dtype != MSA_F32 && dtype != MSA_BF16) || !block_ok(block) || !topk_ok(topk) ||
      !prefill_shape_ok(q_pos0, n_q, hq, d, block, topk) || hkv < 1 || hkv > kMaxGridY ||
      hq % hkv != 0 || !std::isfinite(scale) || q_pos0 + n_q > kv_stride ||
      !pairs_ok(n_q, topk))
    return MSA_ERR_INVALID_ARG;
  if (!msa::prefill_supported(dtype, d, hq / hkv)) return MSA_ERR_UNSUPPORTED;
  if (n_q == 0) return MSA_OK;
  if (ws_bytes < msa::prefill_ws_bytes(dtype, q_pos0, n_q, hq, d, block, topk))
    return MSA_ERR_WORKSPACE;
  return status_of(msa::launch_prefill(q, k, v, dtype, kv_stride, q_pos0, n_q,
                                       hq, hkv, d, block, sel, topk, row_ptr,
                                       q_list, slot, scale, o, lse, ws,
                                       as_stream(stream)));
}

int msa_sparse_gqa_prefill_paged(const void *q, const void *k_pages, const void *v_pages,
                                 int64_t n_pages, const int32_t *block_table,
                                 int32_t max_blocks, int64_t q_pos0, int64_t n_q, int32_t hq,
                                 int32_t hkv, int32_t d, int32_t block, const int32_t *sel,
                                 int32_t topk, const int32_t *row_ptr, const int32_t *q_list,
                                 const int32_t *slot, float scale, float *o, float *lse,
                                 void *ws, size_t ws_bytes, void *stream) {
  if (!q || !k_pages || !v_pages || !block_table || !sel || !row_ptr || !q_list || !slot ||
      !o || !ws || n_pages < 1 || max_blocks < 1 || !block_ok(block) || !topk_ok(topk) ||
      !prefill_shape_ok(q_pos0, n_q, hq, d, block, topk) || hkv < 1 || hkv > kMaxGridY ||
      hq % hkv != 0 || !std::isfinite(scale) || !pairs_ok(n_q, topk) ||
      cdiv(q_pos0 + n_q, block) > max_blocks || n_pages > kMaxTokens / block ||
      !bytes_fit((__int128)n_pages * hkv * block * d * 2))
    return MSA_ERR_INVALID_ARG;
  if (!msa::mfma_prefill_supported(MSA_BF16, d, hq / hkv)) return MSA_ERR_UNSUPPORTED;
  if (n_q == 0) return MSA_OK;
  if (ws_bytes < msa::prefill_ws_bytes(MSA_BF16, q_pos0, n_q, hq, d, block, topk))
    return MSA_ERR_WORKSPACE;
  return status_of(msa::launch_prefill_paged(q, k_pages, v_pages, n_pages, block_table, q_pos0,
                                             n_q, hq, hkv, d, block, sel, topk, row_ptr, q_list,
                                             slot, scale, o, lse, ws, as_stream(stream)));
}

// ---------------------------------------------------------------------------
// Several sequences in one call.  bf16 with d = 128 (the matrix-core path):
// the sequences go in chains of at most 64 (and at most kChainBytes of
// workspace, a single larger sequence making a chain of its own), each chain
// one launch sequence over all its sequences -- pool, top-K, CSR inversion and
// sparse attention with merge -- with every sequence's blocks numbered in
// one global CSR.  Other types and head sizes: the single-sequence path per
// sequence, in order, sharing one workspace (stream order makes the reuse
// safe).
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kChainBytes = size_t(16) << 30;

bool varlen_lens_ok(int32_t n_seq, const int64_t *cu_q, const int64_t *cu_kv) {
  if (!cu_q || !cu_kv || n_seq < 1 || n_seq > kMaxGridY || cu_q[0] != 0 || cu_kv[0] != 0)
    return false;
  for (int32_t s = 0; s < n_seq; ++s) {
    // offsets in [0, 2^40] first, so the differences cannot overflow
    if (cu_q[s + 1] < 0 || cu_q[s + 1] > kMaxTokens || cu_kv[s + 1] < 0 ||
        cu_kv[s + 1] > kMaxTokens)
      return false;
    const int64_t qn = cu_q[s + 1] - cu_q[s], kvn = cu_kv[s + 1] - cu_kv[s];
    if (qn < 0 || kvn < 0 || qn > kvn || !pairs_ok(qn, kMaxTopk)) return false;
  }
  return true;
}

bool chain_path(int32_t dtype, int32_t d) { return dtype == MSA_BF16 && d == 128; }

// Sub-buffers of one chain (or, on the per-sequence path, of one sequence).
struct VarlenLayout {
  size_t kmax, row_ptr, q_list, slot, sel_g, inv, attn, total;
};

VarlenLayout make_layout(int64_t nb, int64_t nq, int32_t d_idx, int32_t topk, size_t inv,
                         size_t attn) {
  VarlenLayout L;
  size_t off = 0;
  L.kmax = off;    off += msa::align256((size_t)nb * d_idx * 4);
  L.row_ptr = off; off += msa::align256((size_t)(nb + 1) * 4);
  L.q_list = off;  off += msa::align256((size_t)nq * topk * 4);
  L.slot = off;    off += msa::align256((size_t)nq * topk * 4);
  L.sel_g = off;   off += msa::align256((size_t)nq * topk * 4);
  L.inv = off;     off += msa::align256(std::max<size_t>(inv, 1));
  L.attn = off;    off += msa::align256(std::max<size_t>(attn, 1));
  L.total = off;
  return L;
}

// The table of the sequences [a, e) with queries (empty ones skipped): query
// rows from cu_q[a], K/V rows absolute.
msa::SeqTab chain_tab(const int64_t *cu_q, const int64_t *cu_kv, int32_t a, int32_t e,
                      int32_t block) {
  msa::SeqTab t{};
  t.B = block;
  int n = 0;
  for (int32_t s = a; s < e; ++s) {
    const int64_t qn = cu_q[s + 1] - cu_q[s], kvn = cu_kv[s + 1] - cu_kv[s];
    if (qn == 0) continue;
    t.q_row0[n] = cu_q[s] - cu_q[a];
    t.q_pos0[n] = kvn - qn;
    t.kv_row0[n] = cu_kv[s];
    t.blk0[n + 1] = t.blk0[n] + (int32_t)cdiv(kvn, block);
    t.qt0[n + 1] = t.qt0[n] + (int32_t)cdiv(qn, 64);
    t.ob0[n + 1] = t.ob0[n] + (int32_t)((kvn - 1) / block - (kvn - qn) / block + 1);
    ++n;
    t.q_row0[n] = cu_q[s + 1] - cu_q[a];
    t.kv_row0[n] = cu_kv[s + 1];
  }
  t.n = n;
  return t;
}

VarlenLayout chain_layout(const msa::SeqTab &t, int32_t hq, int32_t d, int32_t d_idx,
                          int32_t topk) {
  const int64_t nb = t.blk0[t.n], nq = t.q_row0[t.n];
  return make_layout(nb, nq, d_idx, topk, msa::invert_ws_bytes(nq, topk, nb),
                     msa::prefill_chain_ws_bytes(t, hq, d, topk));
}

// Calls fn(a, e, table, layout) for each chain, in order.
extern "C++" template <typename F>
void for_each_chain(int32_t n_seq, const int64_t *cu_q, const int64_t *cu_kv, int32_t hq,
                    int32_t d, int32_t d_idx, int32_t block, int32_t topk, F &&fn) {
  int32_t a = 0;
  while (a < n_seq) {
    int32_t e = a, n = 0;
    while (e < n_seq) {
      if (cu_q[e + 1] == cu_q[e]) {
        ++e;
        continue;
      }
      if (n > 0) {
        if (n == msa::kMaxSeqs) break;
        const msa::SeqTab t = chain_tab(cu_q, cu_kv, a, e + 1, block);
        if (!pairs_ok(t.q_row0[t.n], topk) || t.blk0[t.n] >= INT32_MAX / 2 ||
            chain_layout(t, hq, d, d_idx, topk).total > kChainBytes)
          break;
      }
      ++e;
      ++n;
    }
    const msa::SeqTab t = chain_tab(cu_q, cu_kv, a, e, block);
    if (t.n > 0) fn(a, e, t, chain_layout(t, hq, d, d_idx, topk));
    a = e;
  }
}

VarlenLayout varlen_layout(int32_t dtype, int32_t n_seq, const int64_t *cu_q,
                           const int64_t *cu_kv, int32_t hq, int32_t d, int32_t d_idx,
                           int32_t block, int32_t topk) {
  if (chain_path(dtype, d)) {
    // one layout for every chain: each field sized for the largest chain
    int64_t nb_max = 1, q_max = 1;
    size_t inv = 0, attn = 0;
    for_each_chain(n_seq, cu_q, cu_kv, hq, d, d_idx, block, topk,
                   [&](int32_t, int32_t, const msa::SeqTab &t, const VarlenLayout &) {
                     const int64_t nb = t.blk0[t.n], nq = t.q_row0[t.n];
                     nb_max = std::max(nb_max, nb);
                     q_max = std::max(q_max, nq);
                     inv = std::max(inv, msa::invert_ws_bytes(nq, topk, nb));
                     attn = std::max(attn, msa::prefill_chain_ws_bytes(t, hq, d, topk));
                   });
    return make_layout(nb_max, q_max, d_idx, topk, inv, attn);
  }
  int64_t nb_max = 1, q_max = 1;
  size_t inv = 0, attn = 0;
  for (int32_t s = 0; s < n_seq; ++s) {
    const int64_t qn = cu_q[s + 1] - cu_q[s], kvn = cu_kv[s + 1] - cu_kv[s];
    if (qn == 0) continue;
    const int64_t nb = cdiv(kvn, block);
    nb_max = std::max(nb_max, nb);
    q_max = std::max(q_max, qn);
    inv = std::max(inv, msa::invert_ws_bytes(qn, topk, nb));
    attn = std::max(attn, msa::prefill_ws_bytes(dtype, kvn - qn, qn, hq, d, block, topk));
  }
  return make_layout(nb_max, q_max, d_idx, topk, inv, attn);
}
}  // namespace

size_t msa_prefill_varlen_workspace_bytes(int32_t dtype, int32_t n_seq, const int64_t *cu_q,
                                          const int64_t *cu_kv, int32_t hq, int32_t d,
                                          int32_t d_idx, int32_t block, int32_t topk) {
  if ((dtype != MSA_F32 && dtype != MSA_BF16) || !varlen_lens_ok(n_seq, cu_q, cu_kv) ||
      !prefill_shape_ok(0, cu_kv[n_seq], hq, d, block, kMaxTopk) || !didx_ok(d_idx) ||
      !block_ok(block) || !topk_ok(topk))
    return 0;
  return varlen_layout(dtype, n_seq, cu_q, cu_kv, hq, d, d_idx, block, topk).total;
}

int msa_prefill_varlen(const void *q, const void *k, const void *v, const float *idx_q,
                       const float *idx_k, int32_t dtype, int32_t n_seq, const int64_t *cu_q,
                       const int64_t *cu_kv, int32_t hq, int32_t hkv, int32_t d,
                       int32_t d_idx, int32_t block, int32_t topk, float scale, int32_t *sel,
                       float *o, float *lse, void *ws, size_t ws_bytes, void *stream) {
  if (!q || !k || !v || !idx_q || !idx_k || !sel || !o || !ws ||
      (dtype != MSA_F32 && dtype != MSA_BF16) || !varlen_lens_ok(n_seq, cu_q, cu_kv) ||
      hq < 1 || hkv < 1 || hkv > kMaxGridY || hq % hkv != 0 || d < 1 || !didx_ok(d_idx) ||
      !block_ok(block) || !topk_ok(topk) || !std::isfinite(scale) ||
      !prefill_shape_ok(0, cu_kv[n_seq], hq, d, block, kMaxTopk))
    return MSA_ERR_INVALID_ARG;
  if (!msa::prefill_supported(dtype, d, hq / hkv)) return MSA_ERR_UNSUPPORTED;
  const VarlenLayout L = varlen_layout(dtype, n_seq, cu_q, cu_kv, hq, d, d_idx, block, topk);
  if (ws_bytes < L.total) return MSA_ERR_WORKSPACE;
  char *w = static_cast<char *>(ws);
  float *kmax = reinterpret_cast<float *>(w + L.kmax);
  int32_t *row_ptr = reinterpret_cast<int32_t *>(w + L.row_ptr);
  int32_t *q_list = reinterpret_cast<int32_t *>(w + L.q_list);
  int32_t *slot = reinterpret_cast<int32_t *>(w + L.slot);
  int32_t *sel_g = reinterpret_cast<int32_t *>(w + L.sel_g);
  void *inv_ws = w + L.inv;
  void *attn_ws = w + L.attn;
  const hipStream_t st = as_stream(stream);
  const int64_t es = dtype == MSA_BF16 ? 2 : 4;   // bytes per q/k/v element
  const int64_t total_kv = cu_kv[n_seq];
  if (chain_path(dtype, d)) {
    hipError_t e = hipSuccess;
    for_each_chain(n_seq, cu_q, cu_kv, hq, d, d_idx, block, topk,
                   [&](int32_t a, int32_t, const msa::SeqTab &t, const VarlenLayout &) {
                     if (e != hipSuccess) return;
                     const int64_t r0 = cu_q[a], nq = t.q_row0[t.n], nb = t.blk0[t.n];
                     int32_t *sel_c = sel + r0 * topk;
                     e = msa::launch_pool_tab(idx_k, t, d_idx, kmax, st);
                     if (e == hipSuccess)
                       e = msa::launch_topk_tab(idx_q + r0 * d_idx, t, kmax, d_idx, topk, 1,
                                                sel_c, sel_g, st);
                     if (e == hipSuccess)
                       e = msa::launch_invert(sel_g, nq, topk, nb, row_ptr, q_list, slot,
                                              inv_ws, st);
                     if (e == hipSuccess)
                       e = msa::launch_prefill_chain(
                           static_cast<const char *>(q) + r0 * hq * d * es, k, v,
                           msa::KvMap{nullptr, 0, total_kv, 0, hkv}, t,
                           hq, hkv, d, sel_c, topk, row_ptr, q_list, slot, scale,
                           o + r0 * hq * d, lse ? lse + r0 * hq : nullptr, attn_ws, st);
                   });
    return e == hipSuccess ? MSA_OK : MSA_ERR_HIP;
  }
  for (int32_t s = 0; s < n_seq; ++s) {
    const int64_t qn = cu_q[s + 1] - cu_q[s], kvn = cu_kv[s + 1] - cu_kv[s];
    if (qn == 0) continue;
    const int64_t q0 = kvn - qn, nb = cdiv(kvn, block);
    const char *qs = static_cast<const char *>(q) + cu_q[s] * hq * d * es;
    const char *ks = static_cast<const char *>(k) + cu_kv[s] * d * es;
    const char *vs = static_cast<const char *>(v) + cu_kv[s] * d * es;
    int32_t *sel_s = sel + cu_q[s] * topk;
    hipError_t e = msa::launch_pool(idx_k + cu_kv[s] * d_idx, 1, kvn, nullptr, d_idx, block, 0,
                                    nb, kmax, nb, st);
    if (e == hipSuccess)
      e = msa::launch_topk_prefill(idx_q + cu_q[s] * d_idx, qn, q0, kmax, nb, d_idx, block,
                                   topk, 1, sel_s, st);
    if (e == hipSuccess)
      e = msa::launch_invert(sel_s, qn, topk, nb, row_ptr, q_list, slot, inv_ws, st);
    if (e == hipSuccess)
      e = msa::launch_prefill(qs, ks, vs, dtype, total_kv, q0, qn, hq, hkv, d, block, sel_s,
                              topk, row_ptr, q_list, slot, scale, o + cu_q[s] * hq * d,
                              lse ? lse + cu_q[s] * hq : nullptr, attn_ws, st);
    if (e != hipSuccess) return MSA_ERR_HIP;
  }
  return MSA_OK;
}

size_t msa_decode_workspace_bytes(int32_t n_seq, int32_t hq, int32_t d,
                                  int32_t block, int32_t topk) {
  if (!block_ok(block) || !topk_ok(topk) || !decode_shape_ok(n_seq, 1, hq, d, block, topk))
    return 0;
  return msa::decode_ws_bytes(n_seq, hq, d, block, topk);
}

int msa_sparse_gqa_decode(const void *q, const void *k_cache,
                          const void *v_cache, int32_t dtype, int32_t n_seq,
                          int64_t len_max, const int64_t *seq_len, int32_t hq,
                          int32_t hkv, int32_t d, int32_t block,
                          const int32_t *sel, int32_t topk, float scale,
                          float *o, float *lse, void *ws, size_t ws_bytes,
                          void *stream) {
  if (!q || !k_cache || !v_cache || !seq_len || !sel || !o || !ws ||
      (dtype != MSA_F32 && dtype != MSA_BF16) || n_seq < 1 ||
      n_seq > kMaxGridY || len_max < 1 || hq < 1 || hkv < 1 ||
      hkv > kMaxGridY || hq % hkv != 0 || d < 1 || !block_ok(block) ||
      !topk_ok(topk) || !std::isfinite(scale) ||
      (int64_t)n_seq * hkv * topk > kMaxDecodeItems ||
      !decode_shape_ok(n_seq, 1, hq, d, block, topk))
    return MSA_ERR_INVALID_ARG;
  if (!msa::decode_supported(dtype, d, hq / hkv) ||
      !msa::decode_partials_ok(dtype, d, hq / hkv, block, topk))
    return MSA_ERR_UNSUPPORTED;
  if (ws_bytes < msa::decode_ws_bytes(n_seq, hq, d, block, topk))
    return MSA_ERR_WORKSPACE;
  return status_of(msa::launch_decode(q, k_cache, v_cache, dtype, n_seq,
                                      len_max, seq_len, hq, hkv, d, block, sel,
                                      topk, scale, o, lse, ws,
                                      as_stream(stream)));
}

int msa_sparse_gqa_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                                int32_t kv_dtype, const float *k_scale,
                                const float *v_scale, int64_t n_pages,
                                const int32_t *block_table, int32_t max_blocks,
                                int32_t n_seq, const int64_t *seq_len, int32_t hq,
                                int32_t hkv, int32_t d, int32_t block,
                                const int32_t *sel, int32_t topk, float scale, float *o,
                                float *lse, void *ws, size_t ws_bytes, void *stream) {
  if (!q || !k_pages || !v_pages || !block_table || !seq_len || !sel || !o || !ws ||
      (kv_dtype == MSA_FP8_E4M3 && (!k_scale || !v_scale)) ||
      (kv_dtype != MSA_BF16 && kv_dtype != MSA_FP8_E4M3) || n_pages < 1 ||
      max_blocks < 1 || n_seq < 1 || n_seq > kMaxGridY || hq < 1 || hkv < 1 ||
      hq % hkv != 0 || d < 1 || !block_ok(block) || !topk_ok(topk) ||
      !std::isfinite(scale) || (int64_t)n_seq * hkv * topk > kMaxDecodeItems ||
      (int64_t)n_pages * hkv * block > (int64_t(1) << 40) ||
      !decode_shape_ok(n_seq, max_blocks, hq, d, block, topk))
    return MSA_ERR_INVALID_ARG;
  if (!msa::decode_paged_supported(kv_dtype, d, hq / hkv)) return MSA_ERR_UNSUPPORTED;
  if (ws_bytes < msa::decode_ws_bytes(n_seq, hq, d, block, topk)) return MSA_ERR_WORKSPACE;
  return status_of(msa::launch_decode_paged(q, k_pages, v_pages, kv_dtype, k_scale, v_scale,
                                            n_pages, block_table, max_blocks, n_seq, seq_len,
                                            hq, hkv, block, sel, topk, scale, o, lse, ws,
                                            as_stream(stream)));
}

size_t msa_decode_step_workspace_bytes(int32_t n_seq, int64_t nb_max, int32_t hq,
                                       int32_t d, int32_t block, int32_t topk) {
  if (!block_ok(block) || !topk_ok(topk) || !decode_shape_ok(n_seq, nb_max, hq, d, block, topk))
    return 0;
  return msa::decode_step_ws_bytes(n_seq, nb_max, hq, d, block, topk);
}

int msa_decode_step(const void *q, const void *k_new, const void *v_new,
                    const float *idx_q, const float *idx_k_new, void *k_cache,
                    void *v_cache, float *idx_k_cache, float *kmax, int32_t dtype,
                    int32_t n_seq, int64_t len_max, int64_t nb_max,
                    const int64_t *seq_len, int32_t hq, int32_t hkv, int32_t d,
                    int32_t d_idx, int32_t block, int32_t topk, float scale,
                    int32_t *sel, float *o, float *lse, void *ws, size_t ws_bytes,
                    void *stream) {
  if (!q || !k_new || !v_new || !idx_q || !idx_k_new || !k_cache || !v_cache || !kmax ||
      !seq_len || !sel || !o || !ws || (dtype != MSA_F32 && dtype != MSA_BF16) ||
      n_seq < 1 || n_seq > kMaxGridY || len_max < 1 || nb_max < 1 ||
      nb_max > INT32_MAX || hq < 1 || hkv < 1 || hq % hkv != 0 || d < 1 ||
      !didx_ok(d_idx) || !block_ok(block) || !topk_ok(topk) || !std::isfinite(scale) ||
      (int64_t)n_seq * hkv * topk > kMaxDecodeItems ||
      !decode_shape_ok(n_seq, nb_max, hq, d, block, topk))
    return MSA_ERR_INVALID_ARG;
  if (!msa::decode_step_supported(dtype, d, hq / hkv)) return MSA_ERR_UNSUPPORTED;
  if (ws_bytes < msa::decode_step_ws_bytes(n_seq, nb_max, hq, d, block, topk))
    return MSA_ERR_WORKSPACE;
  return status_of(msa::launch_decode_step(q, k_new, v_new, idx_q, idx_k_new, k_cache,
                                           v_cache, nullptr, 0, 0, idx_k_cache, kmax, n_seq,
                                           len_max,
                                           nb_max, seq_len, hq, hkv, d, d_idx, block, topk,
                                           scale, sel, o, lse, ws, as_stream(stream)));
}

int msa_decode_step_paged(const void *q, const void *k_new, const void *v_new,
                          const float *idx_q, const float *idx_k_new, void *k_pages,
                          void *v_pages, int64_t n_pages, const int32_t *block_table,
                          int32_t max_blocks, float *idx_k_cache, float *kmax, int32_t n_seq,
                          int64_t len_max, int64_t nb_max, const int64_t *seq_len, int32_t hq,
                          int32_t hkv, int32_t d, int32_t d_idx, int32_t block, int32_t topk,
                          float scale, int32_t *sel, float *o, float *lse, void *ws,
                          size_t ws_bytes, void *stream) {
  if (!q || !k_new || !v_new || !idx_q || !idx_k_new || !k_pages || !v_pages ||
      !block_table || !kmax || !seq_len || !sel || !o || !ws || n_pages < 1 ||
      max_blocks < 1 || n_seq < 1 || n_seq > kMaxGridY || len_max < 1 || nb_max < 1 ||
      nb_max > INT32_MAX || hq < 1 || hkv < 1 || hq % hkv != 0 || d < 1 ||
      !didx_ok(d_idx) || !block_ok(block) || !topk_ok(topk) || !std::isfinite(scale) ||
      (int64_t)n_seq * hkv * topk > kMaxDecodeItems ||
      (int64_t)n_pages * hkv * block > (int64_t(1) << 40) ||
      !decode_shape_ok(n_seq, nb_max, hq, d, block, topk))
    return MSA_ERR_INVALID_ARG;
  if (!msa::decode_step_supported(MSA_BF16, d, hq / hkv)) return MSA_ERR_UNSUPPORTED;
  if (ws_bytes < msa::decode_step_ws_bytes(n_seq, nb_max, hq, d, block, topk))
    return MSA_ERR_WORKSPACE;
  return status_of(msa::launch_decode_step(q, k_new, v_new, idx_q, idx_k_new, k_pages, v_pages,
                                           block_table, max_blocks, n_pages, idx_k_cache,
                                           kmax, n_seq, len_max, nb_max, seq_len, hq, hkv, d,
                                           d_idx, block, topk, scale, sel, o, lse, ws,
                                           as_stream(stream)));
}

size_t msa_decode_step_noalloc_max_bytes(void) { return msa::noalloc_scratch_bytes(); }

int msa_decode_step_noalloc(const void *q, const void *k_new, const void *v_new,
                            const float *idx_q, const float *idx_k_new, void *k_cache,
                            void *v_cache, float *idx_k_cache, float *kmax, int32_t dtype,
                            int32_t n_seq, int64_t len_max, int64_t nb_max,
                            const int64_t *seq_len, int32_t hq, int32_t hkv, int32_t d,
                            int32_t d_idx, int32_t block, int32_t topk, float scale,
                            int32_t *sel, float *o, float *lse, void *stream) {
  if (!q || !k_new || !v_new || !idx_q || !idx_k_new || !k_cache || !v_cache || !kmax ||
      !seq_len || !sel || !o || (dtype != MSA_F32 && dtype != MSA_BF16) ||
      n_seq < 1 || n_seq > kMaxGridY || len_max < 1 || nb_max < 1 ||
      nb_max > INT32_MAX || hq < 1 || hkv < 1 || hq % hkv != 0 || d < 1 ||
      !didx_ok(d_idx) || !block_ok(block) || !topk_ok(topk) || !std::isfinite(scale) ||
      (int64_t)n_seq * hkv * topk > kMaxDecodeItems ||
      !decode_shape_ok(n_seq, nb_max, hq, d, block, topk))
    return MSA_ERR_INVALID_ARG;
  if (!msa::decode_step_supported(dtype, d, hq / hkv)) return MSA_ERR_UNSUPPORTED;
  if (msa::decode_step_ws_bytes(n_seq, nb_max, hq, d, block, topk) >
      msa::noalloc_scratch_bytes())
    return MSA_ERR_WORKSPACE;
  void *ws = nullptr;
  if (msa::noalloc_scratch(&ws) != hipSuccess) return MSA_ERR_HIP;
  return status_of(msa::launch_decode_step(q, k_new, v_new, idx_q, idx_k_new, k_cache,
                                           v_cache, nullptr, 0, 0, idx_k_cache, kmax, n_seq,
                                           len_max,
                                           nb_max, seq_len, hq, hkv, d, d_idx, block, topk,
                                           scale, sel, o, lse, ws, as_stream(stream)));
}

}  // extern "C"

