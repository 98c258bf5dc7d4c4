// seqtab.h -- the sequences of one prefill launch chain.
//
// A chain covers up to kMaxSeqs sequences packed one after another
// (prefill over a batch of requests of different lengths, section 3.3
// "Prefilling 与 Decoding 的差异化优化" of chenxutan.com's "MiniMax M3 深度实战"):
//   queries   rows q_row0[s] .. q_row0[s+1]-1 of the packed query arrays, at
//             positions q_pos0[s] .. of their sequence;
//   K/V       rows kv_row0[s] .. of the [Hkv][kv_stride][d] caches (and of the
//             packed index keys), one per position of the sequence;
//   blocks    global block ids blk0[s] .. blk0[s+1]-1 (local block b of
//             sequence s is blk0[s] + b): the summaries, the CSR rows and the
//             KV-outer work items of all sequences share one numbering;
//   tiles     qt0[s]: first 64-query top-K tile of sequence s; ob0[s]: first
//             of its blocks that hold queries (own-block pass tiles).
// A selection never crosses sequences, so every global CSR row holds the
// queries of one sequence.  A single sequence is the table with n = 1.
// The table travels by value in the kernel arguments.
#pragma once
#include <stdint.h>

namespace msa {

constexpr int kMaxSeqs = 64;

struct SeqTab {
  int32_t n;                        // sequences
  int32_t B;                        // block size
  int64_t q_row0[kMaxSeqs + 1];     // prefix of query counts
  int64_t q_pos0[kMaxSeqs];         // position of each sequence's first query
  int64_t kv_row0[kMaxSeqs + 1];    // first K/V row (prefix of K/V lengths)
  int32_t blk0[kMaxSeqs + 1];       // prefix of block counts ceil((q_pos0 + n_q) / B)
  int32_t qt0[kMaxSeqs + 1];        // prefix of 64-query tile counts
  int32_t ob0[kMaxSeqs + 1];        // prefix of query-holding block counts
};

// Index s with a[s] <= x < a[s+1] among the first n + 1 prefix entries
// (a[0] = 0, x < a[n]); sequences with no entries are skipped.
template <typename T>
__host__ __device__ __forceinline__ int prefix_find(const T *a, int n, int64_t x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)a[mid] <= x)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

__host__ __device__ __forceinline__ int64_t seq_nq(const SeqTab &t, int s) {
  return t.q_row0[s + 1] - t.q_row0[s];
}

// Queries of sequence s (positions q_pos0[s] + i) whose own block is <= the
// local block b, counted from the chain's first query: the CSR entries of
// own blocks in the global rows up to and including blk0[s] + b.
__host__ __device__ __forceinline__ int64_t own_through_g(const SeqTab &t, int s, int64_t b) {
  int64_t x = (b + 1) * (int64_t)t.B;
  const int64_t p0 = t.q_pos0[s], p1 = p0 + seq_nq(t, s);
  if (x < p0) x = p0;
  if (x > p1) x = p1;
  return t.q_row0[s] + (x - p0);
}

// Where a chain's keys and values live.  Contiguous (pages == null): the
// [Hkv][kv_stride][d] caches, sequence s from row kv_row0[s].  Paged: the
// [n_pages][Hkv][B][d] pools, local block b of sequence s in page
// pages[s * pt_stride + b]; an entry outside [0, n_pages) is clamped into
// the pool (nothing outside it is read; the outputs of queries that use such
// a block are then unspecified).
struct KvMap {
  const int32_t *pages;
  int64_t n_pages;
  int64_t kv_stride;
  int32_t pt_stride;
  int32_t hkv;
};

// Element offset (head size D) of key 0 of local block b of sequence s in
// KV head g; the block's keys follow row by row.
template <int D>
__host__ __device__ __forceinline__ int64_t kv_block_off(const KvMap &m, const SeqTab &t, int s,
                                                         int64_t b, int g) {
  if (m.pages) {
    int64_t pg = m.pages[(int64_t)s * m.pt_stride + b];
    pg = pg < 0 ? 0 : (pg >= m.n_pages ? m.n_pages - 1 : pg);
    return ((pg * m.hkv + g) * t.B) * D;
  }
  return ((int64_t)g * m.kv_stride + t.kv_row0[s] + b * t.B) * D;
}

// The table of one sequence: queries at positions q_pos0 .. q_pos0 + n_q - 1,
// K/V rows from 0, blocks 0 .. ceil((q_pos0 + n_q) / B) - 1.
inline SeqTab seqtab_one(int64_t q_pos0, int64_t n_q, int32_t block) {
  SeqTab t{};
  t.n = 1;
  t.B = block;
  t.q_row0[1] = n_q;
  t.q_pos0[0] = q_pos0;
  t.kv_row0[1] = q_pos0 + n_q;
  t.blk0[1] = (int32_t)((q_pos0 + n_q + block - 1) / block);
  t.qt0[1] = (int32_t)((n_q + 63) / 64);
  t.ob0[1] = n_q > 0 ? (int32_t)((q_pos0 + n_q - 1) / block - q_pos0 / block + 1) : 0;
  return t;
}

}  // namespace msa
