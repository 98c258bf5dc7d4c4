// invert.hip -- the queries that hit each KV block, as CSR, built without a
// sort.  The KV-outer loop (section 2.2 "KV Outer Gather Q：MSA 的关键设计" of
// chenxutan.com's "MiniMax M3 深度实战") needs, per block, its queries.
//
// Three kernels, each spread over many workgroups:
//   1. hist     per query tile, per block: hit counts (LDS integer atomics --
//               order-free), written as a [tile][block] table;
//   2. colscan  per group of 16 blocks: the exclusive scan of each block's
//               column over the tiles (each tile's offset inside the block's
//               row, written in place) and the row totals;
//   3. scatter  per tile: the row pointers (an exclusive scan of the totals,
//               redone by every workgroup in LDS; tile 0 also stores them),
//               then the tile's queries in ascending order, 256 at a time:
//               every thread ORs its bit into an LDS bitmap (four 64-bit
//               words, one per wave) for each block it selected, so its rank
//               among the threads that hit the same block is a popcount of the
//               lower bits.  The first such thread then advances that block's
//               cursor.  Rows come out ascending by query; the result is
//               deterministic.
// Blocks are processed in ranges of kNR (LDS capacity), so any block count
// works.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kNR = 2048;     // blocks per LDS range
constexpr int kCG = 16;       // blocks per column-scan workgroup

// Queries per tile: the smallest power of two from 256 to 4096 that keeps the
// tile count at most 1024.
int tile_q(int64_t n_q) {
  int tq = 256;
  while (tq < 4096 && (n_q + tq - 1) / tq > 1024) tq *= 2;
  return tq;
}

__global__ __launch_bounds__(256) void inv_hist(const int32_t *__restrict__ sel,
                                                int64_t n_q, int topk,
                                                int64_t nb, int tq,
                                                int32_t *__restrict__ hist) {
  __shared__ int cnt[kNR];
  const int64_t t = blockIdx.x;
  const int64_t i0 = t * tq;
  const int64_t nt = (n_q - i0 < tq ? n_q - i0 : tq) * topk;
  const int32_t *s = sel + i0 * topk;
  for (int64_t r0 = 0; r0 < nb; r0 += kNR) {
    const int nr = (int)(nb - r0 < kNR ? nb - r0 : kNR);
    for (int j = threadIdx.x; j < nr; j += 256) cnt[j] = 0;
    __syncthreads();
    for (int64_t e = threadIdx.x; e < nt; e += 256) {
      const int32_t b = s[e];
      if (b >= r0 && b < r0 + nr) atomicAdd(&cnt[b - r0], 1);
    }
    __syncthreads();
    for (int j = threadIdx.x; j < nr; j += 256) hist[t * nb + r0 + j] = cnt[j];
    __syncthreads();
  }
}

// Column scan of kCG blocks: thread (j, r) owns block b0 + j and the r-th of
// kR contiguous ranges of tiles.  Pass 1 sums each range (loads batched so
// their round trips overlap); the ranges' sums are scanned in LDS; pass 2
// rewrites each tile's count as its exclusive offset in the block's row.
__global__ __launch_bounds__(256) void inv_colscan(int32_t *__restrict__ hist,
                                                   int64_t n_tiles, int64_t nb,
                                                   int32_t *__restrict__ total) {
  constexpr int kR = 256 / kCG;   // tile ranges per block
  constexpr int kBatch = 16;      // loads in flight per thread
  __shared__ int32_t part[kR][kCG];
  const int j = threadIdx.x % kCG, r = threadIdx.x / kCG;
  const int64_t b = (int64_t)blockIdx.x * kCG + j;
  const bool ok = b < nb;
  const int64_t per = (n_tiles + kR - 1) / kR;
  const int64_t t_lo = r * per, t_hi = t_lo + per < n_tiles ? t_lo + per : n_tiles;
  int32_t sum = 0;
  for (int64_t t0 = t_lo; t0 < t_hi; t0 += kBatch) {
    int32_t h[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t t = t0 + u;
      h[u] = ok && t < t_hi ? hist[t * nb + b] : 0;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) sum += h[u];
  }
  part[r][j] = sum;
  __syncthreads();
  int32_t run = 0;
  for (int q = 0; q < r; ++q) run += part[q][j];
  if (ok && r == kR - 1) total[b] = run + sum;
  for (int64_t t0 = t_lo; t0 < t_hi; t0 += kBatch) {
    int32_t h[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t t = t0 + u;
      h[u] = ok && t < t_hi ? hist[t * nb + b] : 0;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t t = t0 + u;
      if (ok && t < t_hi) hist[t * nb + b] = run;
      run += h[u];
    }
  }
}

__device__ __forceinline__ int32_t block_exclusive_scan_256(int32_t x, int32_t *wsum,
                                                            int32_t &all) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int32_t off = 0;
  for (int w = 0; w < wave; ++w) off += wsum[w];
  all = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  return off + inc - x;
}

__global__ __launch_bounds__(256) void inv_scatter(
    const int32_t *__restrict__ sel, int64_t n_q, int topk, int64_t nb, int tq,
    const int32_t *__restrict__ base, const int32_t *__restrict__ total,
    int32_t *__restrict__ row_ptr, int32_t *__restrict__ q_list,
    int32_t *__restrict__ slot) {
  __shared__ int32_t cursor[kNR];
  __shared__ unsigned long long bits[kNR][4];
  __shared__ int32_t wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t = blockIdx.x;
  const int64_t i0 = t * tq;
  const unsigned long long below = (1ull << lane) - 1ull;
  int32_t carry = 0;   // row pointer of the current range's first block
  for (int64_t r0 = 0; r0 < nb; r0 += kNR) {
    const int nr = (int)(nb - r0 < kNR ? nb - r0 : kNR);
    // row pointers of this range: exclusive scan of the totals, 256 blocks
    // at a time (each thread keeps its blocks' starts in the cursor array)
    for (int c0 = 0; c0 < nr; c0 += 256) {
      const int j = c0 + tid;
      const int32_t x = j < nr ? total[r0 + j] : 0;
      int32_t all;
      const int32_t ex = block_exclusive_scan_256(x, wsum, all);
      if (j < nr) {
        cursor[j] = carry + ex + base[t * nb + r0 + j];
        if (t == 0) {
          row_ptr[r0 + j] = carry + ex;
          if (r0 + j == nb - 1) row_ptr[nb] = carry + ex + x;
        }
        bits[j][0] = bits[j][1] = bits[j][2] = bits[j][3] = 0ull;
      }
      carry += all;
    }
    __syncthreads();
    for (int64_t g0 = i0; g0 < i0 + tq && g0 < n_q; g0 += 256) {
      const int64_t i = g0 + tid;
      const bool act = i < n_q && i < i0 + tq;
      const int32_t *srow = sel + i * topk;
      for (int k = 0; k < topk; ++k) {
        const int32_t b = act ? srow[k] : -1;
        if (b >= r0 && b < r0 + nr) atomicOr(&bits[b - r0][wave], 1ull << lane);
      }
      __syncthreads();
      unsigned long long lead = 0ull;
      for (int k = 0; k < topk; ++k) {
        const int32_t b = act ? srow[k] : -1;
        if (b >= r0 && b < r0 + nr) {
          const unsigned long long *m = bits[b - r0];
          int rank = __popcll(m[wave] & below);
          for (int w = 0; w < wave; ++w) rank += __popcll(m[w]);
          const int32_t pos = cursor[b - r0] + rank;
          q_list[pos] = (int32_t)i;
          slot[i * topk + k] = pos;
          if (rank == 0) lead |= 1ull << k;
        } else if (act && r0 == 0 && b < 0) {
          slot[i * topk + k] = -1;
        }
      }
      __syncthreads();
      for (int k = 0; k < topk; ++k) {
        if (!((lead >> k) & 1ull)) continue;
        const int32_t b = srow[k];
        unsigned long long *m = bits[b - r0];
        cursor[b - r0] += __popcll(m[0]) + __popcll(m[1]) + __popcll(m[2]) + __popcll(m[3]);
        m[0] = m[1] = m[2] = m[3] = 0ull;
      }
      __syncthreads();
    }
  }
}

}  // namespace

size_t invert_ws_bytes(int64_t n_q, int32_t topk, int64_t n_blocks) {
  (void)topk;
  // the most tiles any range of at most n_q queries uses (tile_q grows with
  // the range, so a shorter range can use more tiles than n_q itself)
  const int64_t n_small = (n_q + 255) / 256;
  const int64_t n_tiles_small = n_small < 1024 ? n_small : 1024;
  const int64_t n_tiles_large = (n_q + 4095) / 4096;
  const int64_t n_tiles = n_tiles_small > n_tiles_large ? n_tiles_small : n_tiles_large;
  return align256((size_t)(n_tiles > 0 ? n_tiles : 1) * n_blocks * 4) +
         align256((size_t)n_blocks * 4);
}

hipError_t launch_invert(const int32_t *sel, int64_t n_q, int32_t topk,
                         int64_t n_blocks, int32_t *row_ptr, int32_t *q_list,
                         int32_t *slot, void *ws, hipStream_t st) {
  const int tq = tile_q(n_q);
  const int64_t n_tiles = (n_q + tq - 1) / tq;
  const size_t ws_all = invert_ws_bytes(n_q, topk, n_blocks);
  int32_t *hist = static_cast<int32_t *>(ws);
  int32_t *total = reinterpret_cast<int32_t *>(
      static_cast<char *>(ws) + ws_all - align256((size_t)n_blocks * 4));
  if (n_tiles > 0) {
    hipLaunchKernelGGL(inv_hist, dim3((unsigned)n_tiles), dim3(256), 0, st, sel,
                       n_q, topk, n_blocks, tq, hist);
  }
  hipLaunchKernelGGL(inv_colscan, dim3((unsigned)((n_blocks + kCG - 1) / kCG)),
                     dim3(256), 0, st, hist, n_tiles, n_blocks, total);
  hipLaunchKernelGGL(inv_scatter, dim3((unsigned)(n_tiles > 0 ? n_tiles : 1)), dim3(256), 0,
                     st, sel, n_q, topk, n_blocks, tq, hist, total, row_ptr, q_list, slot);
  return hipGetLastError();
}

}  // namespace msa
