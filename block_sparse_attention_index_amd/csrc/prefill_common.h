// prefill_common.h -- pieces shared by the two sparse-prefill
// implementations (VALU and MFMA): the own-entry count of a CSR row and the
// per-row tile table of the KV-outer pass.
#pragma once
#include "msa_internal.h"
#include "seqtab.h"

namespace msa {

// Queries i in [0, n_q) (positions q_pos0 + i) whose own block is <= b.
__device__ __host__ __forceinline__ int64_t own_through(int64_t b,
                                                       int64_t q_pos0,
                                                       int64_t n_q, int B) {
  int64_t x = (b + 1) * (int64_t)B;
  if (x < q_pos0) x = q_pos0;
  if (x > q_pos0 + n_q) x = q_pos0 + n_q;
  return x - q_pos0;
}

namespace {

// tile_ptr[b] = sum over global rows b' < b of ceil(non-own entries of b' /
// tq), capped at max_tiles (the workspace's tile capacity; a valid CSR never
// reaches it, an invalid one is cut short rather than overrunning it).
__global__ __launch_bounds__(1024) void prefill_tiles(
    const int32_t *__restrict__ row_ptr, SeqTab tab, int tq, int64_t max_tiles,
    int32_t *__restrict__ tile_ptr) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nb = tab.blk0[tab.n];
  if (tid == 0) {
    carry_s = 0;
    tile_ptr[0] = 0;
  }
  __syncthreads();
  for (int64_t base = 0; base < nb; base += 1024) {
    const int64_t b = base + tid;
    int32_t x = 0;
    if (b < nb) {
      const int sq = prefix_find(tab.blk0, tab.n, b);
      const int64_t lb = b - tab.blk0[sq];
      const int64_t own = own_through_g(tab, sq, lb) - own_through_g(tab, sq, lb - 1);
      int64_t non = (int64_t)(row_ptr[b + 1] - row_ptr[b]) - own;
      if (non < 0) non = 0;
      x = (int32_t)((non + tq - 1) / tq);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int32_t off = carry_s;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (b < nb) tile_ptr[b + 1] = off + x < max_tiles ? off + x : (int32_t)max_tiles;
    __syncthreads();
    if (tid == 1023) carry_s = off + x;
    __syncthreads();
  }
}

// Row b with tile_ptr[b] <= w < tile_ptr[b+1].
__device__ __forceinline__ int64_t find_row(const int32_t *tile_ptr,
                                            int64_t nb, int64_t w) {
  int64_t lo = 0, hi = nb - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (tile_ptr[mid] <= w)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

}  // namespace
}  // namespace msa
