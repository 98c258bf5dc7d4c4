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
// ballot (its rank) and one lane shift.  Cross-lane reads here are
// v_readlane (a wave-uniform source lane) and DPP moves, never LDS permutes.
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

// Value of lane `src`, src the same in every lane (v_readlane: no LDS trip).
__device__ __forceinline__ float lane_f(float x, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), src));
}
__device__ __forceinline__ int lane_i(int x, int src) {
  return __builtin_amdgcn_readlane(x, src);
}
// Value of lane l-1 (lane 0 keeps its own): a DPP wave_shr:1 move.
__device__ __forceinline__ int prev_lane_i(int x) {
  return __builtin_amdgcn_update_dpp(x, x, 0x138, 0xF, 0xF, false);
}
__device__ __forceinline__ float prev_lane_f(float x) {
  return __int_as_float(prev_lane_i(__float_as_int(x)));
}

// Insert the lanes of `mask` (candidates s at block base+lane) into the
// list (ls, lb) of length *cnt <= km held in lanes [0, km).
__device__ __forceinline__ void list_insert(float s, int base, uint64_t mask,
                                            int km, int &cnt, float &ls,
                                            int &lb) {
  const int lane = threadIdx.x & 63;
  while (mask) {
    const int src = __ffsll((unsigned long long)mask) - 1;
    const float sj = lane_f(s, src);
    const int bj = base + src;
    const int pos = __popcll(__ballot(lane < cnt && ls >= sj));
    const float ps = prev_lane_f(ls);
    const int pb = prev_lane_i(lb);
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
    const float thr = lane_f(ls, km - 1);
    mask &= ~(1ull << src);
    mask &= __ballot(cnt < km || s > thr);
  }
}

// Write sel row: the cnt list blocks ascending, then the forced blocks
// first .. own (own alone without a local window), then -1.  The list blocks
// all lie below `first`, so the row is ascending.
__device__ __forceinline__ void write_row(int32_t *row, int topk, int cnt,
                                          int lb, int own, int first) {
  const int lane = threadIdx.x & 63;
  int rank = 0;
  for (int j = 0; j < cnt; ++j) {
    const int bj = lane_i(lb, j);
    rank += (bj < lb) ? 1 : 0;
  }
  const int nf = own - first + 1;
  if (lane < cnt) row[rank] = lb;
  if (lane >= cnt && lane < cnt + nf) row[lane] = first + (lane - cnt);
  if (lane >= cnt + nf && lane < topk) row[lane] = -1;
}
__device__ __forceinline__ void write_row(int32_t *row, int topk, int cnt,
                                          int lb, int own) {
  write_row(row, topk, cnt, lb, own, own);
}

// First block of the forced local window of `win` blocks ending at `own`.
__device__ __forceinline__ int window_first(int own, int win) {
  return own - win + 1 > 0 ? own - win + 1 : 0;
}

constexpr int kDecChunk = 64;    // blocks per decode-scan workgroup

// As list_insert, with explicit per-lane block ids.
__device__ __forceinline__ void list_insert_ids(float s, int bid, uint64_t mask,
                                                int km, int &cnt, float &ls,
                                                int &lb) {
  const int lane = threadIdx.x & 63;
  while (mask) {
    const int src = __ffsll((unsigned long long)mask) - 1;
    const float sj = lane_f(s, src);
    const int bj = lane_i(bid, src);
    const int pos = __popcll(__ballot(lane < cnt && ls >= sj));
    const float ps = prev_lane_f(ls);
    const int pb = prev_lane_i(lb);
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
    const float thr = lane_f(ls, km - 1);
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

// Candidate key for the merge: an unsigned integer pair ordered like (score
// descending, block ascending) -- hi is the score's order-preserving image
// (-0 counted as +0, so equal scores tie as floats do), lo the complement of
// the block id; (0, 0) stands for "no candidate".
__device__ __forceinline__ uint32_t cand_hi(float s) {
  return (uint32_t)f2key(s == 0.f ? 0.f : s) ^ 0x80000000u;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t x) {
  const uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
  return x > y ? x : y;
}

// Wave-wide unsigned maximum (every lane must be active): DPP steps within
// each 16-lane row (quad swaps, half-row and row mirrors), then the four row
// maxima read as scalars.  The result is uniform.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = dpp_max_u32<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  x = dpp_max_u32<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x = dpp_max_u32<0x141>(x);   // row_half_mirror
  x = dpp_max_u32<0x140>(x);   // row_mirror
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}

// Wave-wide best key (hi first, then lo): two maxima, the second over the
// lanes that hold the best hi.  Uniform result.
__device__ __forceinline__ void wave_max_key(uint32_t &hi, uint32_t &lo) {
  const uint32_t h = wave_max_u32(hi);
  lo = wave_max_u32(hi == h ? lo : 0u);
  hi = h;
}

// Decode index scan, one workgroup (256 threads) per chunk of kDecChunk = 64
// blocks of one sequence: 16 lanes per block row, each taking 8 consecutive
// index columns per 128-column slice (two 16-byte loads), four rows per
// 16-lane group, the partial dot products reduced within the group.  The
// loads depend only on nb_max, not on `own`, so they can be in flight before
// the sequence length arrives.  The chunk's best km among the candidate
// blocks b < cand_lim (score desc, block asc) are then picked by one wave, one
// candidate per lane, in km rounds of a wave-wide maximum, and written in that
// order to (out_s, out_b), the tail padded with (-inf, -1).  (Without a local
// window cand_lim is the own block and km = K-1.)
__device__ __forceinline__ void decode_scan_chunk(
    const float *__restrict__ qv, const float *__restrict__ kmax_s, int64_t cand_lim,
    int64_t nb_max, int d_idx, int km, int ch, float *__restrict__ out_s,
    int *__restrict__ out_b) {
  constexpr int kPass = kDecChunk / 16;
  __shared__ float scs[kDecChunk];
  const int tid = threadIdx.x;
  const int r0 = tid >> 4, l16 = tid & 15;   // first row of the lane group, lane in it
  const int64_t cb0 = (int64_t)ch * kDecChunk;
  const int64_t av = nb_max - cb0;
  const int avail = av < 0 ? 0 : (av > kDecChunk ? kDecChunk : (int)av);
  float acc[kPass];
#pragma unroll
  for (int p = 0; p < kPass; ++p) acc[p] = 0.f;
  if ((d_idx & 7) == 0) {
    for (int c0 = 8 * l16; c0 < d_idx; c0 += 128) {
      const float4 q0 = *reinterpret_cast<const float4 *>(qv + c0);
      const float4 q1 = *reinterpret_cast<const float4 *>(qv + c0 + 4);
      float4 x0[kPass], x1[kPass];
#pragma unroll
      for (int p = 0; p < kPass; ++p) {
        const int r = r0 + 16 * p;
        x0[p] = make_float4(0.f, 0.f, 0.f, 0.f);
        x1[p] = x0[p];
        if (r < avail) {
          const float *row = kmax_s + (cb0 + r) * d_idx + c0;
          x0[p] = *reinterpret_cast<const float4 *>(row);
          x1[p] = *reinterpret_cast<const float4 *>(row + 4);
        }
      }
#pragma unroll
      for (int p = 0; p < kPass; ++p) {
        float a = acc[p];
        a = fmaf(x0[p].x, q0.x, a);
        a = fmaf(x0[p].y, q0.y, a);
        a = fmaf(x0[p].z, q0.z, a);
        a = fmaf(x0[p].w, q0.w, a);
        a = fmaf(x1[p].x, q1.x, a);
        a = fmaf(x1[p].y, q1.y, a);
        a = fmaf(x1[p].z, q1.z, a);
        a = fmaf(x1[p].w, q1.w, a);
        acc[p] = a;
      }
    }
  } else {
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int r = r0 + 16 * p;
      if (r < avail) {
        const float *row = kmax_s + (cb0 + r) * d_idx;
        for (int c = l16; c < d_idx; c += 16) acc[p] = fmaf(row[c], qv[c], acc[p]);
      }
    }
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1)
#pragma unroll
    for (int p = 0; p < kPass; ++p) acc[p] += __shfl_xor(acc[p], o, 64);
  int64_t lim = cand_lim < nb_max ? cand_lim : nb_max;   // candidates are a prefix
  lim -= cb0;
  const int nv = lim < 0 ? 0 : (lim > kDecChunk ? kDecChunk : (int)lim);
  if (l16 == 0)
#pragma unroll
    for (int p = 0; p < kPass; ++p) scs[r0 + 16 * p] = acc[p];
  __syncthreads();
  if (km > 0 && tid < 64) {
    // one candidate per lane; K-1 rounds each take the wave's best key
    static_assert(kDecChunk == 64, "one scan candidate per lane");
    const int j = tid;
    const float sj = scs[j];
    uint32_t kh = j < nv ? cand_hi(sj) : 0u;
    uint32_t kl = j < nv ? ~(uint32_t)(cb0 + j) : 0u;
    for (int r = 0; r < km; ++r) {
      uint32_t h = kh, l = kl;
      wave_max_key(h, l);
      const bool mine = kh == h && kl == l && (h | l) != 0u;
      if (mine) {
        out_s[r] = sj;
        out_b[r] = (int)~l;
        kh = 0u;
        kl = 0u;
      }
      if ((h | l) == 0u && j == 0) {   // fewer than K-1 candidates: pad
        out_s[r] = -INFINITY;
        out_b[r] = -1;
      }
    }
  }
}

// Merge of at most 64 chunk lists of length km <= KM, one whole wave: lane c
// keeps chunk c's list in registers as keys; each of the K-1 rounds takes the
// wave-wide best head and the winning lane shifts its list up.  The winners
// are uniform, so the ascending row is ranked without any exchange.
template <int KM, typename OwnF>
__device__ __forceinline__ void merge_lists_regs(const float *__restrict__ g_s,
                                                 const int *__restrict__ g_b, int n_chunks,
                                                 int km, int topk, int win, OwnF own_f,
                                                 int32_t *row) {
  const int lane = threadIdx.x & 63;
  const bool has = lane < n_chunks;
  uint32_t kh[KM], kl[KM];
#pragma unroll
  for (int i = 0; i < KM; ++i) {
    float sv = 0.f;
    int bv = -1;
    if (has && i < km) {
      sv = g_s[(int64_t)lane * km + i];
      bv = g_b[(int64_t)lane * km + i];
    }
    kh[i] = bv >= 0 ? cand_hi(sv) : 0u;
    kl[i] = bv >= 0 ? ~(uint32_t)bv : 0u;
  }
  uint32_t wins[KM];
  int cnt = 0;
  bool done = false;
#pragma unroll
  for (int r = 0; r < KM; ++r) {
    wins[r] = 0u;
    if (r < km && !done) {
      uint32_t h = kh[0], l = kl[0];
      wave_max_key(h, l);
      if ((h | l) == 0u) {
        done = true;   // every list exhausted
      } else {
        wins[r] = ~l;
        cnt = r + 1;
        if (kh[0] == h && kl[0] == l) {   // this lane's head won: shift its list
#pragma unroll
          for (int i = 0; i + 1 < KM; ++i) {
            kh[i] = kh[i + 1];
            kl[i] = kl[i + 1];
          }
          kh[KM - 1] = 0u;
          kl[KM - 1] = 0u;
        }
      }
    }
  }
  const int own = own_f();
  int mine = INT32_MAX, rank = 0;
#pragma unroll
  for (int i = 0; i < KM; ++i)
    if (i < cnt && i == lane) mine = (int)wins[i];
#pragma unroll
  for (int i = 0; i < KM; ++i) rank += (i < cnt && (int)wins[i] < mine) ? 1 : 0;
  const int first = window_first(own, win), nf = own - first + 1;
  if (lane < cnt) row[rank] = mine;
  if (lane >= cnt && lane < cnt + nf) row[lane] = first + (lane - cnt);
  if (lane >= cnt + nf && lane < topk) row[lane] = -1;
}

// Decode merge, one whole wave: the per-chunk lists of one sequence (each
// sorted, score descending, padded with id -1, km = K - win entries) into the
// selection row: the best km blocks ascending, then the forced window
// own-win+1 .. own (clipped at block 0), then -1.  Up to 64 lists of up to 15
// entries merge in registers (above); up to 256 lists take a K-1-round
// tournament over the list heads: lane c holds the heads of chunks c, c+64,
// c+128, c+192, a round takes the wave-wide best head and advances that list.
// `row` may point to LDS.  More than 256 chunks fall back to inserting the
// candidates one by one into a running list.  `own_f()` gives the own block;
// it is called only after the lists' loads are issued (so a length it reads
// can be in flight with them).
constexpr int kMergeLanesChunks = 4;   // chunk lists per lane in the tournament

template <typename OwnF>
__device__ __forceinline__ void decode_merge_lists(
    const float *__restrict__ g_s, const int *__restrict__ g_b, int n_chunks, int topk,
    int win, OwnF own_f, int32_t *row, float *stage_s = nullptr, int *stage_b = nullptr,
    int stage_cap = 0) {
  const int lane = threadIdx.x & 63;
  const int km = topk - win;   // picks by score; lists hold km entries each
  if (km > 0 && n_chunks <= 64 && km <= 7) {
    merge_lists_regs<7>(g_s, g_b, n_chunks, km, topk, win, own_f, row);
    return;
  }
  if (km > 0 && n_chunks <= 64 && km <= 15) {
    merge_lists_regs<15>(g_s, g_b, n_chunks, km, topk, win, own_f, row);
    return;
  }
  // copy the lists to the caller's LDS scratch when they fit: the tournament
  // then reads each advanced head at LDS latency
  const float *in_s = g_s;
  const int *in_b = g_b;
  const int64_t n_cand = (int64_t)n_chunks * (km > 0 ? km : 0);
  if (stage_s && n_cand <= stage_cap) {
    constexpr int kBatch = 16;   // loads per lane in flight together
    for (int64_t i0 = 0; i0 < n_cand; i0 += 64 * kBatch) {
      float xs[kBatch];
      int xb[kBatch];
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        const int64_t i = i0 + 64 * t + lane;
        xs[t] = i < n_cand ? g_s[i] : 0.f;
        xb[t] = i < n_cand ? g_b[i] : 0;
      }
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        const int64_t i = i0 + 64 * t + lane;
        if (i < n_cand) {
          stage_s[i] = xs[t];
          stage_b[i] = xb[t];
        }
      }
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
    const int own = own_f();
    write_row(row, topk, cnt, lane < cnt ? tops : INT32_MAX, own, window_first(own, win));
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
      const float thr = lane_f(ls, km - 1);
      const uint64_t mask = __ballot(xbs[gi] >= 0 && (cnt < km || xs[gi] > thr));
      if (mask) list_insert_ids(xs[gi], xbs[gi], mask, km, cnt, ls, lb);
    }
  }
  if (lane >= cnt) lb = INT32_MAX;
  const int own = own_f();
  write_row(row, topk, cnt, lb, own, window_first(own, win));
}

}  // namespace msa
