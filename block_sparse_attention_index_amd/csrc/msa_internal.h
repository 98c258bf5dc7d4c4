// msa_internal.h -- declarations shared by the host entry points and the
// gfx950 kernels of the MSA library (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "seqtab.h"

namespace msa {

// Launch helpers: each enqueues its kernels on `st` and returns the HIP
// status of the launch.  Arguments were validated by the entry point.

hipError_t launch_pool_mean(const float *idx_k, int32_t n_seq, int64_t len_max,
                            const int64_t *seq_len, int32_t d_idx, int32_t block,
                            int64_t blk_begin, int64_t blk_end, float *kmean,
                            int64_t nb_max, hipStream_t st);
hipError_t launch_pool(const float *idx_k, int32_t n_seq, int64_t len_max,
                       const int64_t *seq_len, int32_t d_idx, int32_t block,
                       int64_t blk_begin, int64_t blk_end, float *kmax,
                       int64_t nb_max, hipStream_t st);

hipError_t launch_topk_prefill(const float *idx_q, int64_t n_q, int64_t q_pos0,
                               const float *kmax, int64_t nb, int32_t d_idx,
                               int32_t block, int32_t topk, int32_t win, int32_t *sel,
                               hipStream_t st);

// Chain-table forms (sequences packed one after another, see seqtab.h):
// the max-pool of every global block, and the per-query top-K of every
// sequence (sel: local block ids; sel_g, if not null: global ids).
hipError_t launch_pool_tab(const float *idx_k, const SeqTab &tab, int32_t d_idx, float *kmax,
                           hipStream_t st);
hipError_t launch_topk_tab(const float *idx_q, const SeqTab &tab, const float *kmax,
                           int32_t d_idx, int32_t topk, int32_t win, int32_t *sel,
                           int32_t *sel_g, hipStream_t st);

size_t topk_decode_ws_bytes(int32_t n_seq, int64_t nb_max, int32_t topk);
size_t topk_batch_ws_bytes(int64_t n_q, int64_t nb_max, int32_t topk);
hipError_t launch_topk_batch(const float *idx_q, int64_t n_q, const int32_t *q_seq,
                             const int64_t *q_pos, const float *kmax, int32_t n_seq,
                             int64_t nb_max, int32_t d_idx, int32_t block, int32_t topk,
                             int32_t *sel, void *ws, hipStream_t st);
hipError_t launch_topk_decode(const float *idx_q, int32_t n_seq,
                              const int64_t *seq_len, const float *kmax,
                              int64_t nb_max, int32_t d_idx, int32_t block,
                              int32_t topk, int32_t win, int32_t *sel, void *ws,
                              hipStream_t st);

size_t invert_ws_bytes(int64_t n_q, int32_t topk, int64_t n_blocks);
hipError_t launch_invert(const int32_t *sel, int64_t n_q, int32_t topk,
                         int64_t n_blocks, int32_t *row_ptr, int32_t *q_list,
                         int32_t *slot, void *ws, hipStream_t st);

// Number of (query, block) pairs whose block is not the query's own block,
// for queries at positions [q_pos0, q_pos0 + n_q): a closed form, since every
// query keeps min(K, own + 1) blocks.
int64_t nonown_pairs(int64_t q_pos0, int64_t n_q, int32_t block, int32_t topk);

size_t prefill_ws_bytes(int32_t dtype, int64_t q_pos0, int64_t n_q, int32_t hq,
                        int32_t d, int32_t block, int32_t topk);
bool prefill_supported(int32_t dtype, int32_t d, int32_t group);
hipError_t launch_prefill(const void *q, const void *k, const void *v,
                          int32_t dtype, int64_t kv_stride, int64_t q_pos0,
                          int64_t n_q, int32_t hq, int32_t hkv, int32_t d,
                          int32_t block, const int32_t *sel, int32_t topk,
                          const int32_t *row_ptr, const int32_t *q_list,
                          const int32_t *slot, float scale, float *o,
                          float *lse, void *ws, hipStream_t st);

// The matrix-core sparse prefill (bf16, d = 128) over the sequences of one
// chain table (queries packed by sequence, K/V rows at tab.kv_row0[s]): the
// workspace it needs and its launch.  The CSR is global over the table's
// blocks.
size_t prefill_chain_ws_bytes(const SeqTab &tab, int32_t hq, int32_t d, int32_t topk);
hipError_t launch_prefill_chain(const void *q, const void *k, const void *v,
                                const KvMap &kvm, const SeqTab &tab, int32_t hq,
                                int32_t hkv, int32_t d, const int32_t *sel, int32_t topk,
                                const int32_t *row_ptr, const int32_t *q_list,
                                const int32_t *slot, float scale, float *o, float *lse,
                                void *ws, hipStream_t st);

// The matrix-core sparse prefill of one sequence over a paged bf16 cache
// (block b in page block_table[b]; pages [n_pages][Hkv][B][d]).
hipError_t launch_prefill_paged(const void *q, const void *k_pages, const void *v_pages,
                                int64_t n_pages, const int32_t *block_table, int64_t q_pos0,
                                int64_t n_q, int32_t hq, int32_t hkv, int32_t d, int32_t block,
                                const int32_t *sel, int32_t topk, const int32_t *row_ptr,
                                const int32_t *q_list, const int32_t *slot, float scale,
                                float *o, float *lse, void *ws, hipStream_t st);

size_t decode_ws_bytes(int32_t n_seq, int32_t hq, int32_t d, int32_t block,
                       int32_t topk);
bool decode_supported(int32_t dtype, int32_t d, int32_t group);
bool decode_partials_ok(int32_t dtype, int32_t d, int32_t group, int32_t block,
                        int32_t topk);
hipError_t launch_decode(const void *q, const void *k_cache,
                         const void *v_cache, int32_t dtype, int32_t n_seq,
                         int64_t len_max, const int64_t *seq_len, int32_t hq,
                         int32_t hkv, int32_t d, int32_t block,
                         const int32_t *sel, int32_t topk, float scale,
                         float *o, float *lse, void *ws, hipStream_t st);

bool decode_paged_supported(int32_t kv_dtype, int32_t d, int32_t group);
hipError_t launch_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                               int32_t kv_dtype, const float *k_scale, const float *v_scale,
                               int64_t n_pages, const int32_t *block_table, int32_t max_blocks,
                               int32_t n_seq, const int64_t *seq_len, int32_t hq, int32_t hkv,
                               int32_t block, const int32_t *sel, int32_t topk, float scale,
                               float *o, float *lse, void *ws, hipStream_t st);
size_t decode_step_ws_bytes(int32_t n_seq, int64_t nb_max, int32_t hq, int32_t d,
                            int32_t block, int32_t topk);
bool decode_step_supported(int32_t dtype, int32_t d, int32_t group);
// ptab: null for contiguous [n_seq][Hkv][len_max][d] caches, else the
// [n_seq][pt_stride] block table of [n_pages][Hkv][B][d] page pools.
hipError_t launch_decode_step(const void *q, const void *k_new, const void *v_new,
                              const float *idx_q, const float *idx_k_new, void *k_cache,
                              void *v_cache, const int32_t *ptab, int32_t pt_stride,
                              int64_t n_pages, float *idx_k_cache, float *kmax,
                              int32_t n_seq, int64_t len_max, int64_t nb_max,
                              const int64_t *seq_len, int32_t hq, int32_t hkv, int32_t d,
                              int32_t d_idx, int32_t block, int32_t topk, float scale,
                              int32_t *sel, float *o, float *lse, void *ws,
                              hipStream_t st);

// The static scratch of msa_decode_step_noalloc: its size, and its device
// address on the current device (looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void **ptr);

// Round a byte count up to the 256-byte alignment used for workspace
// sub-buffers.
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace msa

// ---------------------------------------------------------------------------
// Device helpers.
// ---------------------------------------------------------------------------
#ifdef __HIPCC__
namespace msa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Wave64 reductions (butterfly over all 64 lanes; every lane gets the result).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Hardware base-2 exponential (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

}  // namespace msa
#endif
