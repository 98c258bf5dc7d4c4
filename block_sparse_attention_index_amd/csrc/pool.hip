// pool.hip -- block max-pool of the single-head index key (index branch of
// "MiniMax M3模型算力成本大幅降低原因深度解析", paragraph "索引分支（Index Branch）").
//
// One workgroup per (block, sequence).  The block's rows are streamed with
// coalesced 16-byte loads (256 threads = R row-groups x d_idx/4 column lanes),
// reduced in registers, then across row-groups through LDS.  The max runs on
// an order-preserving integer image of the float bits, which makes it exact,
// order-free and puts -0 below +0.  HBM-bound: each index key is read once.
#include "msa_internal.h"
#include "index_common.h"

namespace msa {
namespace {

// Max over tokens [t0, t1) of the [*, d_idx] rows at src into dst[d_idx],
// by the whole workgroup.  VEC4: d_idx % 4 == 0 and d_idx <= 1024 (16-byte
// loads, 256 / (d_idx / 4) row groups); else d_idx <= 256.
template <bool VEC4>
__device__ __forceinline__ void pool_rows(const float *__restrict__ src, int64_t t0,
                                          int64_t t1, int d_idx, float *__restrict__ dst) {
  __shared__ int4 red[256];
  const int cw = VEC4 ? d_idx >> 2 : d_idx;   // column lanes
  const int R = 256 / cw;
  const int tid = threadIdx.x;
  const int col = tid % cw, r = tid / cw;
  int4 m = make_int4(INT32_MIN, INT32_MIN, INT32_MIN, INT32_MIN);
  if (r < R) {
    for (int64_t t = t0 + r; t < t1; t += R) {
      if constexpr (VEC4) {
        const float4 x = reinterpret_cast<const float4 *>(src + t * d_idx)[col];
        m.x = max(m.x, f2key(x.x));
        m.y = max(m.y, f2key(x.y));
        m.z = max(m.z, f2key(x.z));
        m.w = max(m.w, f2key(x.w));
      } else {
        m.x = max(m.x, f2key(src[t * d_idx + col]));
      }
    }
  }
  red[tid] = m;
  __syncthreads();
  if (tid < cw) {
    for (int rr = 1; rr < R; ++rr) {
      const int4 y = red[rr * cw + tid];
      m.x = max(m.x, y.x);
      m.y = max(m.y, y.y);
      m.z = max(m.z, y.z);
      m.w = max(m.w, y.w);
    }
    if constexpr (VEC4)
      reinterpret_cast<float4 *>(dst)[tid] =
          make_float4(key2f(m.x), key2f(m.y), key2f(m.z), key2f(m.w));
    else
      dst[tid] = key2f(m.x);
  }
}

// One workgroup per (block, sequence) of a [n_seq][len_max][d_idx] batch.
template <bool VEC4>
__global__ __launch_bounds__(256) void pool_max(
    const float *__restrict__ idx_k, int64_t len_max,
    const int64_t *__restrict__ seq_len, int d_idx, int B, int64_t blk_begin,
    float *__restrict__ kmax, int64_t nb_max) {
  const int s = blockIdx.y;
  int64_t len = seq_len ? seq_len[s] : len_max;
  if (len > len_max) len = len_max;
  if (len < 1) return;
  const int64_t b = blk_begin < 0 ? (len - 1) / B : blk_begin + blockIdx.x;
  const int64_t t0 = b * B;
  if (t0 >= len || b >= nb_max) return;
  const int64_t t1 = t0 + B < len ? t0 + B : len;
  pool_rows<VEC4>(idx_k + ((int64_t)s * len_max) * d_idx, t0, t1, d_idx,
                  kmax + ((int64_t)s * nb_max + b) * d_idx);
}

// One workgroup per global block of a chain table: the sequences' index keys
// packed one after another (sequence s at row tab.kv_row0[s], its length
// being the position after its last query), the summaries of all sequences
// in one [global block][d_idx] array.
template <bool VEC4>
__global__ __launch_bounds__(256) void pool_max_tab(const float *__restrict__ idx_k,
                                                    SeqTab tab, int d_idx,
                                                    float *__restrict__ kmax) {
  const int64_t gb = blockIdx.x;
  const int sq = prefix_find(tab.blk0, tab.n, gb);
  const int64_t b = gb - tab.blk0[sq];
  const int64_t len = tab.q_pos0[sq] + seq_nq(tab, sq);
  const int64_t t0 = b * tab.B;
  const int64_t t1 = t0 + tab.B < len ? t0 + tab.B : len;
  pool_rows<VEC4>(idx_k + tab.kv_row0[sq] * d_idx, t0, t1, d_idx, kmax + gb * d_idx);
}

// Append mode: the newest token t = len-1 of each sequence either starts its
// block's summary (t % B == 0) or raises the running max in place.  Valid
// when kmax[s][t / B] already holds the max over tokens [t/B*B, t).
__global__ __launch_bounds__(256) void pool_append(
    const float *__restrict__ idx_k, int64_t len_max,
    const int64_t *__restrict__ seq_len, int d_idx, int B,
    float *__restrict__ kmax, int64_t nb_max) {
  const int s = blockIdx.x;
  int64_t len = seq_len ? seq_len[s] : len_max;
  if (len > len_max) len = len_max;
  if (len < 1) return;
  const int64_t t = len - 1, b = t / B;
  if (b >= nb_max) return;
  const float *src = idx_k + ((int64_t)s * len_max + t) * d_idx;
  float *dst = kmax + ((int64_t)s * nb_max + b) * d_idx;
  const bool first = (t % B) == 0;
  for (int c = threadIdx.x; c < d_idx; c += 256) {
    const int x = f2key(src[c]);
    dst[c] = first ? src[c] : key2f(max(x, f2key(dst[c])));
  }
}

// Mean-pool variant (the block summary of section 3.3's sketch in
// chenxutan.com's page): kmean[s][b][c] = (sum over the block's valid tokens
// of idx_k[s][t][c]) / count, summed in fp32 -- per thread over rows r,
// r+R, ..., then the R partial sums in row-group order -- and divided once.
// Same grid and row split as the max-pool kernels; d_idx <= 1024 with
// d_idx % 4 == 0, else d_idx <= 256.
template <bool VEC4>
__global__ __launch_bounds__(256) void pool_mean(
    const float *__restrict__ idx_k, int64_t len_max,
    const int64_t *__restrict__ seq_len, int d_idx, int B, int64_t blk_begin,
    float *__restrict__ kmean, int64_t nb_max) {
  __shared__ float4 red[256];
  const int s = blockIdx.y;
  int64_t len = seq_len ? seq_len[s] : len_max;
  if (len > len_max) len = len_max;
  if (len < 1) return;
  const int64_t b = blk_begin < 0 ? (len - 1) / B : blk_begin + blockIdx.x;
  const int64_t t0 = b * B;
  if (t0 >= len || b >= nb_max) return;
  const int64_t t1 = t0 + B < len ? t0 + B : len;
  const int cw = VEC4 ? d_idx >> 2 : d_idx;   // column lanes
  const int R = 256 / cw;
  const int tid = threadIdx.x;
  const int col = tid % cw, r = tid / cw;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  if (r < R) {
    const float *src = idx_k + ((int64_t)s * len_max) * d_idx;
    for (int64_t t = t0 + r; t < t1; t += R) {
      if constexpr (VEC4) {
        const float4 x = reinterpret_cast<const float4 *>(src + t * d_idx)[col];
        a.x += x.x;
        a.y += x.y;
        a.z += x.z;
        a.w += x.w;
      } else {
        a.x += src[t * d_idx + col];
      }
    }
  }
  red[tid] = a;
  __syncthreads();
  if (tid < cw) {
    float4 m = red[tid];
    for (int rr = 1; rr < R; ++rr) {
      const float4 y = red[rr * cw + tid];
      m.x += y.x;
      m.y += y.y;
      m.z += y.z;
      m.w += y.w;
    }
    const float n = (float)(t1 - t0);
    float *dst = kmean + ((int64_t)s * nb_max + b) * d_idx;
    if constexpr (VEC4)
      reinterpret_cast<float4 *>(dst)[tid] = make_float4(m.x / n, m.y / n, m.z / n, m.w / n);
    else
      dst[tid] = m.x / n;
  }
}

}  // namespace

hipError_t launch_pool_mean(const float *idx_k, int32_t n_seq, int64_t len_max,
                            const int64_t *seq_len, int32_t d_idx, int32_t block,
                            int64_t blk_begin, int64_t blk_end, float *kmean,
                            int64_t nb_max, hipStream_t st) {
  const int64_t nblk = blk_begin < 0 ? 1 : blk_end - blk_begin;
  dim3 grid((unsigned)nblk, (unsigned)n_seq);
  if (d_idx % 4 == 0)
    hipLaunchKernelGGL(pool_mean<true>, grid, dim3(256), 0, st, idx_k, len_max, seq_len,
                       d_idx, block, blk_begin, kmean, nb_max);
  else
    hipLaunchKernelGGL(pool_mean<false>, grid, dim3(256), 0, st, idx_k, len_max, seq_len,
                       d_idx, block, blk_begin, kmean, nb_max);
  return hipGetLastError();
}

hipError_t launch_pool(const float *idx_k, int32_t n_seq, int64_t len_max,
                       const int64_t *seq_len, int32_t d_idx, int32_t block,
                       int64_t blk_begin, int64_t blk_end, float *kmax,
                       int64_t nb_max, hipStream_t st) {
  if (blk_begin == -2) {
    hipLaunchKernelGGL(pool_append, dim3((unsigned)n_seq), dim3(256), 0, st,
                       idx_k, len_max, seq_len, d_idx, block, kmax, nb_max);
    return hipGetLastError();
  }
  const int64_t nblk = blk_begin < 0 ? 1 : blk_end - blk_begin;
  dim3 grid((unsigned)nblk, (unsigned)n_seq);
  if (d_idx % 4 == 0)
    hipLaunchKernelGGL(pool_max<true>, grid, dim3(256), 0, st, idx_k, len_max,
                       seq_len, d_idx, block, blk_begin, kmax, nb_max);
  else
    hipLaunchKernelGGL(pool_max<false>, grid, dim3(256), 0, st, idx_k, len_max,
                       seq_len, d_idx, block, blk_begin, kmax, nb_max);
  return hipGetLastError();
}

hipError_t launch_pool_tab(const float *idx_k, const SeqTab &tab, int32_t d_idx, float *kmax,
                           hipStream_t st) {
  const int64_t nb = tab.blk0[tab.n];
  if (nb <= 0) return hipSuccess;
  if (d_idx % 4 == 0)
    hipLaunchKernelGGL(pool_max_tab<true>, dim3((unsigned)nb), dim3(256), 0, st, idx_k, tab,
                       d_idx, kmax);
  else
    hipLaunchKernelGGL(pool_max_tab<false>, dim3((unsigned)nb), dim3(256), 0, st, idx_k, tab,
                       d_idx, kmax);
  return hipGetLastError();
}

}  // namespace msa
