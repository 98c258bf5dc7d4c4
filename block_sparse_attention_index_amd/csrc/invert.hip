// invert.hip -- the queries that hit each KV block, as CSR, built without a
// sort.  The KV-outer loop (section 2.2 "KV Outer Gather Q：MSA 的关键设计" of
// chenxutan.com's "MiniMax M3 深度实战") needs, per block, its queries.
//
//   1. hist     per query tile (1024 queries), per block: hit counts
//               (LDS integer atomics -- order-free);
//   2. colscan  per block, exclusive scan over tiles -> each tile's base
//               offset inside the block's row, and the row total;
//   3. rowptr   exclusive scan of the totals -> row_ptr;
//   4. scatter  one wave per tile walks its queries in ascending order, 64 at
//               a time: every lane ORs its bit into an LDS bitmap word per
//               block it selected, so a lane's rank among the lanes that hit
//               the same block is a popcount of the lower bits.  The lowest
//               such lane then advances that block's cursor.  Rows come out
//               ascending by query and the result is deterministic.
// Blocks are processed in ranges of 4096 (LDS capacity), so any block count
// works.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kNR = 4096;   // blocks per LDS range

// Queries per tile: the smallest power of two from 64 to 1024 that keeps the
// tile count at most 256, so that a short query range still spreads over many
// workgroups (each tile's scatter walks its queries 64 at a time).
int tile_q(int64_t n_q) {
  int tq = 64;
  while (tq < 1024 && (n_q + tq - 1) / tq > 256) tq *= 2;
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

__global__ __launch_bounds__(256) void inv_colscan(int32_t *__restrict__ hist,
                                                   int64_t n_tiles, int64_t nb,
                                                   int32_t *__restrict__ total) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nb) return;
  int32_t run = 0;
  for (int64_t t = 0; t < n_tiles; ++t) {
    const int32_t h = hist[t * nb + b];
    hist[t * nb + b] = run;
    run += h;
  }
  total[b] = run;
}

__global__ __launch_bounds__(1024) void inv_rowptr(const int32_t *__restrict__ total,
                                                   int64_t nb,
                                                   int32_t *__restrict__ row_ptr) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    carry_s = 0;
    row_ptr[0] = 0;
  }
  __syncthreads();
  for (int64_t base = 0; base < nb; base += 1024) {
    const int64_t b = base + tid;
    int32_t x = b < nb ? total[b] : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int32_t off = carry_s;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (b < nb) row_ptr[b + 1] = off + x;
    __syncthreads();
    if (tid == 1023) carry_s = off + x;
    __syncthreads();
  }
}

__global__ __launch_bounds__(64) void inv_scatter(
    const int32_t *__restrict__ sel, int64_t n_q, int topk, int64_t nb, int tq,
    const int32_t *__restrict__ base, const int32_t *__restrict__ row_ptr,
    int32_t *__restrict__ q_list, int32_t *__restrict__ slot) {
  __shared__ int32_t cursor[kNR];
  __shared__ unsigned long long bits[kNR];
  const int lane = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int64_t i0 = t * tq;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int64_t r0 = 0; r0 < nb; r0 += kNR) {
    const int nr = (int)(nb - r0 < kNR ? nb - r0 : kNR);
    for (int j = lane; j < nr; j += 64) {
      cursor[j] = row_ptr[r0 + j] + base[t * nb + r0 + j];
      bits[j] = 0ull;
    }
    __syncthreads();
    for (int sub = 0; sub < tq / 64; ++sub) {
      const int64_t i = i0 + sub * 64 + lane;
      if (i0 + sub * 64 >= n_q) break;
      const bool act = i < n_q;
      const int32_t *srow = sel + i * topk;
      for (int k = 0; k < topk; ++k) {
        const int32_t b = act ? srow[k] : -1;
        if (b >= r0 && b < r0 + nr) atomicOr(&bits[b - r0], 1ull << lane);
      }
      __syncthreads();
      unsigned long long lead = 0ull;
      for (int k = 0; k < topk; ++k) {
        const int32_t b = act ? srow[k] : -1;
        if (b >= r0 && b < r0 + nr) {
          const unsigned long long m = bits[b - r0];
          const int rank = __popcll(m & below);
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
        cursor[b - r0] += __popcll(bits[b - r0]);
        bits[b - r0] = 0ull;
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
  const int64_t n_small = (n_q + 63) / 64;
  const int64_t n_tiles_small = n_small < 256 ? n_small : 256;
  const int64_t n_tiles_large = (n_q + 1023) / 1024;
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
  hipLaunchKernelGGL(inv_colscan, dim3((unsigned)((n_blocks + 255) / 256)),
                     dim3(256), 0, st, hist, n_tiles, n_blocks, total);
  hipLaunchKernelGGL(inv_rowptr, dim3(1), dim3(1024), 0, st, total, n_blocks,
                     row_ptr);
  if (n_tiles > 0) {
    hipLaunchKernelGGL(inv_scatter, dim3((unsigned)n_tiles), dim3(64), 0, st,
                       sel, n_q, topk, n_blocks, tq, hist, row_ptr, q_list, slot);
  }
  return hipGetLastError();
}

}  // namespace msa
