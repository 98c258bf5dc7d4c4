// topk.hip -- q.blockmax scores and per-query causal top-K (index branch of
// "MiniMax M3模型算力成本大幅降低原因深度解析", paragraph "索引分支（Index Branch）";
// prefill scores every earlier block for every query, decode only the new
// query: section 3.3 of chenxutan.com's "MiniMax M3 深度实战").
//
// Selection rule: candidates are the blocks strictly before the query's own
// block; keep the best K-1 by (score desc, block asc); add the own block;
// store ascending, -1 padded.
//
// Running top list, one per query: lanes 0..K-2 of a wave hold the list
// entries in rank order.  Candidates arrive in ascending block order, so a
// candidate enters only if it beats the current (K-1)-th score strictly (an
// equal score already in the list has a lower block index); a ballot picks
// the lanes that beat the threshold, and each is inserted with one more
// ballot (its rank) and one lane shift.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kQT = 64;     // queries per workgroup (prefill)
constexpr int kCB = 64;     // blocks per chunk
constexpr int kDC = 64;     // index columns per staged slice
constexpr int kPad = kDC + 1;
constexpr int kMaxList = 64;

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

// ---------------------------------------------------------------------------
// Prefill: workgroup = 64 consecutive queries; loop over chunks of 64 blocks
// below the workgroup's last own block.  Scores by a 4x4 register tile per
// thread over LDS-staged slices of 64 index columns; then each wave merges 16
// queries' 64 new scores into their lists.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void topk_prefill_kernel(
    const float *__restrict__ idx_q, int64_t n_q, int64_t q_pos0,
    const float *__restrict__ kmax, int d_idx, int B, int topk,
    int32_t *__restrict__ sel) {
  __shared__ float qs[kQT][kPad];
  __shared__ float ks[kCB][kPad];
  __shared__ float lst_s[kQT][kMaxList];
  __shared__ int lst_b[kQT][kMaxList];
  __shared__ int lst_n[kQT];
  float(*sc)[kPad] = qs;  // scores alias the query slice (phases are fenced)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Heavier (later) tiles first.
  const int64_t n_tiles = (n_q + kQT - 1) / kQT;
  const int64_t tile = n_tiles - 1 - blockIdx.x;
  const int64_t q0 = tile * kQT;
  const int nq = (int)(n_q - q0 < kQT ? n_q - q0 : kQT);
  const int km = topk - 1;
  const int64_t own_last = (q_pos0 + q0 + nq - 1) / B;

  if (tid < kQT) lst_n[tid] = 0;
  for (int e = tid; e < kQT * kMaxList; e += 256) {
    lst_s[e / kMaxList][e % kMaxList] = -INFINITY;
    lst_b[e / kMaxList][e % kMaxList] = -1;
  }
  __syncthreads();

  const int ty = tid >> 4, tx = tid & 15;
  for (int64_t b0 = 0; km > 0 && b0 < own_last; b0 += kCB) {
    const int nbk = (int)(own_last - b0 < kCB ? own_last - b0 : kCB);
    float acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[a][c] = 0.f;
    for (int c0 = 0; c0 < d_idx; c0 += kDC) {
      const int dc = d_idx - c0 < kDC ? d_idx - c0 : kDC;
      __syncthreads();
      for (int e = tid; e < kQT * kDC; e += 256) {
        const int r = e / kDC, c = e % kDC;
        qs[r][c] = (r < nq && c < dc) ? idx_q[(q0 + r) * d_idx + c0 + c] : 0.f;
        ks[r][c] = (r < nbk && c < dc) ? kmax[(b0 + r) * d_idx + c0 + c] : 0.f;
      }
      __syncthreads();
      for (int c = 0; c < dc; ++c) {
        float qv[4], kv[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) qv[a] = qs[ty + 16 * a][c];
#pragma unroll
        for (int j = 0; j < 4; ++j) kv[j] = ks[tx + 16 * j][c];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[a][j] = fmaf(qv[a], kv[j], acc[a][j]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[ty + 16 * a][tx + 16 * j] = acc[a][j];
    __syncthreads();
    // Merge: wave w owns queries 16w .. 16w+15.
    for (int jq = 0; jq < 16; ++jq) {
      const int qi = wave * 16 + jq;
      if (qi >= nq) break;
      const int64_t own = (q_pos0 + q0 + qi) / B;
      const float s = sc[qi][lane];
      const bool valid = lane < nbk && b0 + lane < own;
      int cnt = lst_n[qi];
      float ls = lane < km ? lst_s[qi][lane] : -INFINITY;
      int lb = lane < km ? lst_b[qi][lane] : -1;
      const float thr = shfl_f(ls, km - 1);
      const uint64_t mask = __ballot(valid && (cnt < km || s > thr));
      if (mask) {
        list_insert(s, (int)b0, mask, km, cnt, ls, lb);
        if (lane < km) {
          lst_s[qi][lane] = ls;
          lst_b[qi][lane] = lb;
        }
        if (lane == 0) lst_n[qi] = cnt;
      }
    }
  }
  __syncthreads();
  for (int jq = 0; jq < 16; ++jq) {
    const int qi = wave * 16 + jq;
    if (qi >= nq) break;
    const int own = (int)((q_pos0 + q0 + qi) / B);
    const int cnt = km > 0 ? lst_n[qi] : 0;
    const int lb = (lane < cnt) ? lst_b[qi][lane] : INT32_MAX;
    write_row(sel + (q0 + qi) * topk, topk, cnt, lb, own);
  }
}

// ---------------------------------------------------------------------------
// Decode, stage 1: workgroup = (chunk of 64 blocks, sequence).  Each wave
// scores 16 blocks, two at a time (a half-wave reads one summary row with
// 16-byte loads and reduces the dot product across its 32 lanes); wave 0 then
// keeps the chunk's best K-1 and writes them (score desc) to the workspace.
// Stage 2 (one wave per sequence) merges the chunk lists in chunk order, 64
// candidates per ballot, and writes the selection.
// ---------------------------------------------------------------------------
constexpr int kDecChunk = 64;

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

__global__ __launch_bounds__(256) void topk_decode_kernel(
    const float *__restrict__ idx_q, const int64_t *__restrict__ seq_len,
    const float *__restrict__ kmax, int64_t nb_max, int d_idx, int B, int topk,
    float *__restrict__ ws_s, int *__restrict__ ws_b, int n_chunks) {
  __shared__ float scs[kDecChunk];
  const int s = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int km = topk - 1;
  const int64_t len = seq_len[s];
  const int64_t own = len >= 1 ? (len - 1) / B : 0;
  const float *qv = idx_q + (int64_t)s * d_idx;

  // scores of blocks ch*64 + wave*16 + 2*it + (lane >> 5)
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t bw = (int64_t)ch * kDecChunk + wave * 16 + half;
  if ((d_idx & 3) == 0 && d_idx <= 128) {
    // one float4 of the row per lane: all eight row loads in flight at once
    const bool has = 4 * l32 < d_idx;
    const float4 qa = has ? *reinterpret_cast<const float4 *>(qv + 4 * l32)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 x[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {       // issued before own is known
      const int64_t b = bw + 2 * it;
      x[it] = (has && b < nb_max)
                  ? *reinterpret_cast<const float4 *>(
                        kmax + ((int64_t)s * nb_max + b) * d_idx + 4 * l32)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      float acc = qa.x * x[it].x;
      acc = fmaf(qa.y, x[it].y, acc);
      acc = fmaf(qa.z, x[it].z, acc);
      acc = fmaf(qa.w, x[it].w, acc);
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
      const int64_t b = bw + 2 * it;
      if (l32 == 0) scs[wave * 16 + 2 * it + half] = (b < own && b < nb_max) ? acc : -INFINITY;
    }
  } else {
    for (int it = 0; it < 8; ++it) {
      const int64_t b = bw + 2 * it;
      float acc = 0.f;
      const bool valid = b < own && b < nb_max;
      if (valid) {
        const float *row = kmax + ((int64_t)s * nb_max + b) * d_idx;
        for (int c = l32; c < d_idx; c += 32) acc = fmaf(row[c], qv[c], acc);
      }
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
      if (l32 == 0) scs[wave * 16 + 2 * it + half] = valid ? acc : -INFINITY;
    }
  }
  __syncthreads();
  if (wave == 0 && km > 0) {
    const int64_t bb = (int64_t)ch * kDecChunk + lane;
    const float x = scs[lane];
    const bool valid = bb < own && bb < nb_max;
    int cnt = 0;
    float ls = -INFINITY;
    int lb = -1;
    const uint64_t mask = __ballot(valid);
    list_insert(x, ch * kDecChunk, mask, km, cnt, ls, lb);
    const int64_t o = ((int64_t)s * n_chunks + ch) * km;
    if (lane < km) {
      ws_s[o + lane] = lane < cnt ? ls : -INFINITY;
      ws_b[o + lane] = lane < cnt ? lb : -1;
    }
  }
}

__global__ __launch_bounds__(64) void topk_decode_merge(
    const int64_t *__restrict__ seq_len, int B, int topk,
    const float *__restrict__ ws_s, const int *__restrict__ ws_b, int n_chunks,
    int32_t *__restrict__ sel) {
  const int s = blockIdx.x, lane = threadIdx.x;
  const int km = topk - 1;
  const int64_t len = seq_len[s];
  const int64_t own = len >= 1 ? (len - 1) / B : 0;
  int cnt = 0;
  float ls = -INFINITY;
  int lb = INT32_MAX;
  const int64_t nc = (int64_t)n_chunks * km;
  const int64_t o0 = (int64_t)s * n_chunks * km;
  constexpr int kPre = 8;   // candidate groups of 64 fetched in one round trip
  for (int64_t base0 = 0; km > 0 && base0 < nc; base0 += 64 * kPre) {
    float xs[kPre];
    int xbs[kPre];
#pragma unroll
    for (int gi = 0; gi < kPre; ++gi) {
      const int64_t i = base0 + 64 * gi + lane;
      xs[gi] = i < nc ? ws_s[o0 + i] : -INFINITY;
      xbs[gi] = i < nc ? ws_b[o0 + i] : -1;
    }
#pragma unroll
    for (int gi = 0; gi < kPre; ++gi) {
      const float thr = shfl_f(ls, km - 1);
      const uint64_t mask = __ballot(xbs[gi] >= 0 && (cnt < km || xs[gi] > thr));
      if (mask) list_insert_ids(xs[gi], xbs[gi], mask, km, cnt, ls, lb);
    }
  }
  if (lane >= cnt) lb = INT32_MAX;
  write_row(sel + (int64_t)s * topk, topk, cnt, lb, (int)own);
}

}  // namespace

hipError_t launch_topk_prefill(const float *idx_q, int64_t n_q, int64_t q_pos0,
                               const float *kmax, int64_t nb, int32_t d_idx,
                               int32_t block, int32_t topk, int32_t *sel,
                               hipStream_t st) {
  (void)nb;
  const int64_t n_tiles = (n_q + kQT - 1) / kQT;
  hipLaunchKernelGGL(topk_prefill_kernel, dim3((unsigned)n_tiles), dim3(256), 0,
                     st, idx_q, n_q, q_pos0, kmax, d_idx, block, topk, sel);
  return hipGetLastError();
}

// Layout: [chunk scores][chunk block ids].
size_t topk_decode_ws_bytes(int32_t n_seq, int64_t nb_max, int32_t topk) {
  const int64_t n_chunks = (nb_max + kDecChunk - 1) / kDecChunk;
  const size_t n = (size_t)n_seq * n_chunks * (topk > 1 ? topk - 1 : 1);
  return align256(n * sizeof(float)) + align256(n * sizeof(int));
}

hipError_t launch_topk_decode(const float *idx_q, int32_t n_seq,
                              const int64_t *seq_len, const float *kmax,
                              int64_t nb_max, int32_t d_idx, int32_t block,
                              int32_t topk, int32_t *sel, void *ws,
                              hipStream_t st) {
  const int n_chunks = (int)((nb_max + kDecChunk - 1) / kDecChunk);
  const size_t n = (size_t)n_seq * n_chunks * (topk > 1 ? topk - 1 : 1);
  char *w = static_cast<char *>(ws);
  float *ws_s = reinterpret_cast<float *>(w);
  w += align256(n * sizeof(float));
  int *ws_b = reinterpret_cast<int *>(w);
  if (topk > 1) {
    hipLaunchKernelGGL(topk_decode_kernel, dim3(n_chunks, n_seq), dim3(256), 0, st,
                       idx_q, seq_len, kmax, nb_max, d_idx, block, topk, ws_s,
                       ws_b, n_chunks);
  }
  hipLaunchKernelGGL(topk_decode_merge, dim3(n_seq), dim3(64), 0, st, seq_len,
                     block, topk, ws_s, ws_b, n_chunks, sel);
  return hipGetLastError();
}

}  // namespace msa
