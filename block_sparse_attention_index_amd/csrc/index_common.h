// index_common.h -- device pieces of the index branch shared by the top-K
// kernels and the fused decode step ("MiniMax M3模型算力成本大幅降低原因深度解析",
// paragraph "索引分支（Index Branch）"; decode: section 3.3 of chenxutan.com's
// "MiniMax M3 深度实战").
//
// Running top list, one per query: lanes 0..K-2 of a wave hold the list
// entries in rank order.  Candidates arrive in ascending block order, so a
// candidate enters only if it beats the current (K-1)-th score strictly (an
// equal score already in the list has a lower block index); a ballot picks
// the lanes that beat the threshold, and each is inserted with one more
// ballot (its rank) and one lane shift.
#pragma once
#include "msa_internal.h"

namespace msa {

// Order-preserving integer image of a float's bits (exact max, -0 < +0).
__device__ __forceinline__ int f2key(float x) {
  int i = __float_as_int(x);
  return i ^ ((i >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float key2f(int k) {
  return __int_as_float(k ^ ((k >> 31) & 0x7fffffff));
}

__device__ __forceinline__ float shfl_f(float x, int src) {
  return __shfl(x, src, 64);
}
__device__ __forceinline__ int shfl_i(int x, int src) {
  return __shfl(x, src, 64);
}

// Insert the lanes of `mask` (candidates s at block base+lane) into the
// list (ls, lb) of length *cnt <= km held in lanes [0, km).
__device__ __forceinline__ void list_insert(float s, int base, uint64_t mask,
                                            int km, int &cnt, float &ls,
                                            int &lb) {
  const int lane = threadIdx.x & 63;
  while (mask) {
    const int src = __ffsll((unsigned long long)mask) - 1;
    const float sj = shfl_f(s, src);
    const int bj = base + src;
    const int pos = __popcll(__ballot(lane < cnt && ls >= sj));
    const float ps = shfl_f(ls, lane > 0 ? lane - 1 : 0);
    const int pb = shfl_i(lb, lane > 0 ? lane - 1 : 0);
    const int last = cnt < km - 1 ? cnt : km - 1;
    if (lane > pos && lane <= last) {
      ls = ps;
      lb = pb;
    }
    if (lane == pos) {
      ls = sj;
      lb = bj;
    }
    cnt = cnt + 1 < km ? cnt + 1 : km;
    const float thr = shfl_f(ls, km - 1);
    mask &= ~(1ull << src);
    mask &= __ballot(cnt < km || s > thr);
  }
}

// Write sel row: the cnt list blocks ascending, then own, then -1.
__device__ __forceinline__ void write_row(int32_t *row, int topk, int cnt,
                                          int lb, int own) {
  const int lane = threadIdx.x & 63;
  int rank = 0;
  for (int j = 0; j < cnt; ++j) {
    const int bj = shfl_i(lb, j);
    rank += (bj < lb) ? 1 : 0;
  }
  if (lane < cnt) row[rank] = lb;
  if (lane == cnt) row[cnt] = own;
  if (lane > cnt && lane < topk) row[lane] = -1;
}

constexpr int kDecChunk = 16;    // blocks per decode-scan workgroup

// As list_insert, with explicit per-lane block ids.
__device__ __forceinline__ void list_insert_ids(float s, int bid, uint64_t mask,
                                                int km, int &cnt, float &ls,
                                                int &lb) {
  const int lane = threadIdx.x & 63;
  while (mask) {
    const int src = __ffsll((unsigned long long)mask) - 1;
    const float sj = shfl_f(s, src);
    const int bj = shfl_i(bid, src);
    const int pos = __popcll(__ballot(lane < cnt && ls >= sj));
    const float ps = shfl_f(ls, lane > 0 ? lane - 1 : 0);
    const int pb = shfl_i(lb, lane > 0 ? lane - 1 : 0);
    const int last = cnt < km - 1 ? cnt : km - 1;
    if (lane > pos && lane <= last) {
      ls = ps;
      lb = pb;
    }
    if (lane == pos) {
      ls = sj;
      lb = bj;
    }
    cnt = cnt + 1 < km ? cnt + 1 : km;
    const float thr = shfl_f(ls, km - 1);
    mask &= ~(1ull << src);
    mask &= __ballot(cnt < km || s > thr);
  }
}

// Best (score desc, block asc) over the wave's 64 (score, block) pairs; every
// lane receives it.
__device__ __forceinline__ void wave_best(float &s, int &id) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float s2 = __shfl_xor(s, o, 64);
    const int i2 = __shfl_xor(id, o, 64);
    if (s2 > s || (s2 == s && i2 < id)) {
      s = s2;
      id = i2;
    }
  }
}

// Decode index scan, one workgroup (256 threads) per chunk of kDecChunk = 16
// blocks of one sequence (many small workgroups: the scan is latency-bound):
// 16 lanes per block, each taking 8 consecutive index columns of the summary
// row per 128-column slice (two 16-byte loads), the partial dot products
// reduced within the 16-lane row.  The chunk's best K-1 among the blocks
// before `own` are found by rank -- each candidate counts the candidates
// ahead of it (score desc, block asc) -- and written at that rank to (out_s,
// out_b), the tail padded with (-inf, -1).
__device__ __forceinline__ void decode_scan_chunk(
    const float *__restrict__ qv, const float *__restrict__ kmax_s, int64_t own,
    int64_t nb_max, int d_idx, int topk, int ch, float *__restrict__ out_s,
    int *__restrict__ out_b) {
  __shared__ float scs[kDecChunk];
  const int tid = threadIdx.x;
  const int km = topk - 1;
  const int r = tid >> 4, l16 = tid & 15;   // block of the chunk, lane in its row
  int64_t lim = own < nb_max ? own : nb_max;   // valid blocks are a prefix
  lim -= (int64_t)ch * kDecChunk;
  const int nv = lim < 0 ? 0 : (lim > kDecChunk ? kDecChunk : (int)lim);
  const int64_t b = (int64_t)ch * kDecChunk + r;
  float acc = 0.f;
  if (r < nv) {
    const float *row = kmax_s + b * d_idx;
    if ((d_idx & 7) == 0) {
      for (int c0 = 8 * l16; c0 < d_idx; c0 += 128) {
        const float4 x0 = *reinterpret_cast<const float4 *>(row + c0);
        const float4 x1 = *reinterpret_cast<const float4 *>(row + c0 + 4);
        const float4 q0 = *reinterpret_cast<const float4 *>(qv + c0);
        const float4 q1 = *reinterpret_cast<const float4 *>(qv + c0 + 4);
        acc = fmaf(x0.x, q0.x, acc);
        acc = fmaf(x0.y, q0.y, acc);
        acc = fmaf(x0.z, q0.z, acc);
        acc = fmaf(x0.w, q0.w, acc);
        acc = fmaf(x1.x, q1.x, acc);
        acc = fmaf(x1.y, q1.y, acc);
        acc = fmaf(x1.z, q1.z, acc);
        acc = fmaf(x1.w, q1.w, acc);
      }
    } else {
      for (int c = l16; c < d_idx; c += 16) acc = fmaf(row[c], qv[c], acc);
    }
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (l16 == 0) scs[r] = acc;
  __syncthreads();
  if (km > 0 && tid < 64) {
    const int j = tid;
    const float sj = j < nv ? scs[j] : 0.f;
    if (j < nv) {
      int rank = 0;
#pragma unroll
      for (int i = 0; i < kDecChunk; ++i) {
        const float si = scs[i];
        rank += (i < nv && (si > sj || (si == sj && i < j))) ? 1 : 0;
      }
      if (rank < km) {
        out_s[rank] = sj;
        out_b[rank] = (int)((int64_t)ch * kDecChunk + j);
      }
    }
    if (j >= nv && j < km) {
      out_s[j] = -INFINITY;
      out_b[j] = -1;
    }
  }
}

// Decode merge, one wave: the per-chunk lists of one sequence (each sorted,
// score descending, padded with id -1) into the selection row: the best K-1
// blocks ascending, then `own`, then -1.  A K-1-round tournament over the
// list heads: lane c holds the heads of chunks c, c+64, c+128, c+192, a round
// takes the wave-wide best head and advances that list.  `row` may point to
// LDS.  More than 256 chunks fall back to inserting the candidates one by one
// into a running list.
constexpr int kMergeLanesChunks = 4;   // chunk lists per lane in the tournament

__device__ __forceinline__ void decode_merge_lists(
    const float *__restrict__ g_s, const int *__restrict__ g_b, int n_chunks, int topk,
    int own, int32_t *row, float *stage_s = nullptr, int *stage_b = nullptr,
    int stage_cap = 0) {
  const int lane = threadIdx.x & 63;
  const int km = topk - 1;
  // copy the lists to the caller's LDS scratch when they fit: the tournament
  // then reads each advanced head at LDS latency
  const float *in_s = g_s;
  const int *in_b = g_b;
  const int64_t n_cand = (int64_t)n_chunks * (km > 0 ? km : 0);
  if (stage_s && n_cand <= stage_cap) {
    for (int64_t i = lane; i < n_cand; i += 64) {
      stage_s[i] = g_s[i];
      stage_b[i] = g_b[i];
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // the wave's LDS writes have landed
    in_s = stage_s;
    in_b = stage_b;
  }
  if (km > 0 && n_chunks <= 64 * kMergeLanesChunks) {
    int ptr[kMergeLanesChunks];
    float hs[kMergeLanesChunks];
    int hb[kMergeLanesChunks];
#pragma unroll
    for (int t = 0; t < kMergeLanesChunks; ++t) {
      const int c = lane + 64 * t;
      ptr[t] = 0;
      const bool has = c < n_chunks;
      hs[t] = has ? in_s[(int64_t)c * km] : -INFINITY;
      hb[t] = has ? in_b[(int64_t)c * km] : -1;
    }
    int tops = INT32_MAX, cnt = 0;
    for (int r = 0; r < km; ++r) {
      // this lane's best head, then the wave's
      float bs = -INFINITY;
      int bid = INT32_MAX, bt = 0;
#pragma unroll
      for (int t = 0; t < kMergeLanesChunks; ++t) {
        const float x = hb[t] >= 0 ? hs[t] : -INFINITY;
        const int i = hb[t] >= 0 ? hb[t] : INT32_MAX;
        if (x > bs || (x == bs && i < bid)) {
          bs = x;
          bid = i;
          bt = t;
        }
      }
      float ws = bs;
      int wid = bid;
      wave_best(ws, wid);
      if (wid == INT32_MAX) break;   // every list exhausted
      if (lane == r) tops = wid;
      ++cnt;
      if (bid == wid) {   // the winning lane advances that list
#pragma unroll
        for (int t = 0; t < kMergeLanesChunks; ++t) {
          if (t == bt) {
            const int c = lane + 64 * t;
            const int p = ++ptr[t];
            hs[t] = p < km ? in_s[(int64_t)c * km + p] : -INFINITY;
            hb[t] = p < km ? in_b[(int64_t)c * km + p] : -1;
          }
        }
      }
    }
    write_row(row, topk, cnt, lane < cnt ? tops : INT32_MAX, own);
    return;
  }
  int cnt = 0;
  float ls = -INFINITY;
  int lb = INT32_MAX;
  const int64_t nc = n_cand;
  constexpr int kPre = 8;   // candidate groups of 64 fetched in one round trip
  for (int64_t base0 = 0; km > 0 && base0 < nc; base0 += 64 * kPre) {
    float xs[kPre];
    int xbs[kPre];
#pragma unroll
    for (int gi = 0; gi < kPre; ++gi) {
      const int64_t i = base0 + 64 * gi + lane;
      xs[gi] = i < nc ? in_s[i] : -INFINITY;
      xbs[gi] = i < nc ? in_b[i] : -1;
    }
#pragma unroll
    for (int gi = 0; gi < kPre; ++gi) {
      const float thr = shfl_f(ls, km - 1);
      const uint64_t mask = __ballot(xbs[gi] >= 0 && (cnt < km || xs[gi] > thr));
      if (mask) list_insert_ids(xs[gi], xbs[gi], mask, km, cnt, ls, lb);
    }
  }
  if (lane >= cnt) lb = INT32_MAX;
  write_row(row, topk, cnt, lb, own);
}

}  // namespace msa
