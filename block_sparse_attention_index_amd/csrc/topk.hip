// topk.hip -- q.blockmax scores and per-query causal top-K (index branch of
// "MiniMax M3模型算力成本大幅降低原因深度解析", paragraph "索引分支（Index Branch）";
// prefill scores every earlier block for every query, decode only the new
// query: section 3.3 of chenxutan.com's "MiniMax M3 深度实战").
//
// Selection rule: candidates are the blocks strictly before the query's own
// block; keep the best K-1 by (score desc, block asc); add the own block;
// store ascending, -1 padded.  With a local window of win blocks (a variant
// after the sliding window of section 3.3's sketch in chenxutan.com's page),
// the own block and the win-1 blocks before it are forced and the best K-win
// of the blocks below them are kept.
//
// Running top list, one per query: lanes 0..K-2 of a wave hold the list
// entries in rank order.  Candidates arrive in ascending block order, so a
// candidate enters only if it beats the current (K-1)-th score strictly (an
// equal score already in the list has a lower block index); a ballot picks
// the lanes that beat the threshold, and each is inserted with one more
// ballot (its rank) and one lane shift.
#include "msa_internal.h"
#include "index_common.h"

namespace msa {
namespace {

constexpr int kQT = 64;     // queries per workgroup (prefill)
constexpr int kCB = 64;     // blocks per chunk
constexpr int kDC = 64;     // index columns per staged slice (d_idx > kDFull)
constexpr int kDFull = 128; // d_idx up to this: the whole row staged at once

typedef float f32x16s __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Prefill: workgroup = 64 consecutive queries (4 waves); loop over chunks of
// 64 blocks below the workgroup's last own block.  Scores on the fp32 matrix
// cores: wave w computes the 32 x 32 quadrant (queries 32*(w/2).., blocks
// 32*(w%2)..) with v_mfma_f32_32x32x2_f32 from LDS-staged rows (fp32 products
// and sums, as a dot product in any summation order).  The query tile is
// staged once when d_idx <= kDFull (else slice by slice with the blocks).
// Then each wave merges 16 queries' 64 new scores into their lists: first,
// for all 16 at once, which queries have a candidate above their list's
// entry threshold; then insertion only for those -- after the first chunks
// most lists are full and few candidates beat them.
//
// LDS rows are padded to an odd stride (kDFull + 1, kDC + 1 floats), so the
// 32 lanes of a half-wave reading one column of 32 rows hit 32 banks.
// KMAX bounds the list length (K - window).
// ---------------------------------------------------------------------------
//
// A launch covers the sequences of a chain table: tile t belongs to the
// sequence s with qt0[s] <= t < qt0[s+1]; its queries are rows q_row0[s] ..
// of idx_q / sel, its summaries rows blk0[s] .. of kmax.  sel receives block
// ids local to the sequence; sel_g (if not null) the same rows with global
// block ids (local + blk0[s], -1 kept).
template <int KMAX, bool FULL>
__global__ __launch_bounds__(256) void topk_prefill_kernel(
    const float *__restrict__ idx_q_all, SeqTab tab, const float *__restrict__ kmax_all,
    int d_idx, int topk, int win, int32_t *__restrict__ sel_all,
    int32_t *__restrict__ sel_g) {
  constexpr int kW = FULL ? kDFull : kDC;   // staged columns
  constexpr int kPad = kW + 1;
  __shared__ float qs[kQT][kPad];
  __shared__ float ks[kCB][kPad];
  __shared__ float lst_s[kQT][KMAX];
  __shared__ int lst_b[kQT][KMAX];
  __shared__ int lst_n[kQT];
  __shared__ float lst_t[kQT];   // entry threshold: the (K-1)-th score, -inf until full
  __shared__ int64_t lst_lim[kQT];   // first block past the query's candidates
  // scores alias the block rows (written after the MFMAs' last read of them,
  // read before the next chunk's staging; both sides fenced)
  float(*sc)[kPad] = ks;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Heavier (later) tiles first.
  const int64_t tile_g = (int64_t)tab.qt0[tab.n] - 1 - blockIdx.x;
  const int sq = prefix_find(tab.qt0, tab.n, tile_g);
  const int64_t tile = tile_g - tab.qt0[sq];
  const int64_t n_q = seq_nq(tab, sq), q_pos0 = tab.q_pos0[sq];
  const int B = tab.B;
  const float *idx_q = idx_q_all + tab.q_row0[sq] * d_idx;
  const float *kmax = kmax_all + (int64_t)tab.blk0[sq] * d_idx;
  int32_t *sel = sel_all + tab.q_row0[sq] * topk;
  const int64_t q0 = tile * kQT;
  const int nq = (int)(n_q - q0 < kQT ? n_q - q0 : kQT);
  const int km = topk - win;   // picks by score; the window win is forced
  // candidates of the tile's last query: the blocks below its window
  const int64_t cand_last = (q_pos0 + q0 + nq - 1) / B - win + 1;
  // 16-byte loads when every row starts 16-byte aligned
  const bool vq = (d_idx & 3) == 0 && (reinterpret_cast<uintptr_t>(idx_q) & 15) == 0;
  const bool vk = (d_idx & 3) == 0 && (reinterpret_cast<uintptr_t>(kmax) & 15) == 0;

  // rows [r0, r0 + nr) x columns [c0, c0 + dc) of a [*, d_idx] fp32 matrix
  // into dst (zero beyond nr / dc, up to kW columns)
  auto stage = [&](float (*dst)[kPad], const float *src, bool vec, int64_t r0, int nr,
                   int c0, int dc) {
    if (vec) {
      constexpr int kV = kW / 4;
      for (int e = tid; e < kQT * kV; e += 256) {
        const int r = e / kV, c = 4 * (e % kV);
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r < nr && c < dc)
          x = *reinterpret_cast<const float4 *>(src + (r0 + r) * d_idx + c0 + c);
        dst[r][c] = x.x;
        dst[r][c + 1] = x.y;
        dst[r][c + 2] = x.z;
        dst[r][c + 3] = x.w;
      }
    } else {
      for (int e = tid; e < kQT * kW; e += 256) {
        const int r = e / kW, c = e % kW;
        dst[r][c] = (r < nr && c < dc) ? src[(r0 + r) * d_idx + c0 + c] : 0.f;
      }
    }
  };

  if (tid < kQT) {
    lst_n[tid] = 0;
    lst_t[tid] = -INFINITY;
    // one 64-bit division per query, not one per query and chunk
    lst_lim[tid] = (q_pos0 + q0 + tid) / B - win + 1;
  }
  for (int e = tid; e < kQT * KMAX; e += 256) {
    lst_s[e / KMAX][e % KMAX] = -INFINITY;
    lst_b[e / KMAX][e % KMAX] = -1;
  }
  if (FULL) stage(qs, idx_q, vq, q0, nq, 0, d_idx);
  __syncthreads();

  const int qw = wave >> 1, bw = wave & 1;
  const int h = lane >> 5, j = lane & 31;
  for (int64_t b0 = 0; km > 0 && b0 < cand_last; b0 += kCB) {
    const int nbk = (int)(cand_last - b0 < kCB ? cand_last - b0 : kCB);
    f32x16s d;
#pragma unroll
    for (int r = 0; r < 16; ++r) d[r] = 0.f;
    for (int c0 = 0; c0 < d_idx; c0 += kW) {
      const int dc = d_idx - c0 < kW ? d_idx - c0 : kW;
      if (!FULL) stage(qs, idx_q, vq, q0, nq, c0, dc);
      stage(ks, kmax, vk, b0, nbk, c0, dc);
      __syncthreads();
      const int dce = (dc + 1) & ~1;   // K = 2 per step; column dc is zero
      for (int kk = 0; kk < dce; kk += 2) {
        const float a = qs[32 * qw + j][kk + h];
        const float b = ks[32 * bw + j][kk + h];
        d = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, d, 0, 0, 0);
      }
      __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[32 * qw + 8 * (r >> 2) + 4 * h + (r & 3)][32 * bw + j] = d[r];
    __syncthreads();
    // Merge: wave w owns queries 16w .. 16w+15.
    uint32_t need = 0;
    uint64_t masks[16];
#pragma unroll
    for (int jq = 0; jq < 16; ++jq) {
      const int qi = wave * 16 + jq;
      const int64_t lim = lst_lim[qi];
      const float s = sc[qi][lane];
      const float t = lst_t[qi];
      const bool valid = qi < nq && lane < nbk && b0 + lane < lim;
      masks[jq] = __ballot(valid && s > t);
      if (masks[jq]) need |= 1u << jq;
    }
    while (need) {
      const int jq = __ffs(need) - 1;
      need &= need - 1;
      const int qi = wave * 16 + jq;
      const float s = sc[qi][lane];
      int cnt = lst_n[qi];
      float ls = lane < km ? lst_s[qi][lane] : -INFINITY;
      int lb = lane < km ? lst_b[qi][lane] : -1;
      uint64_t mask = 0;
#pragma unroll
      for (int x = 0; x < 16; ++x)
        if (x == jq) mask = masks[x];
      list_insert(s, (int)b0, mask, km, cnt, ls, lb);
      if (lane < km) {
        lst_s[qi][lane] = ls;
        lst_b[qi][lane] = lb;
      }
      const float thr = lane_f(ls, km - 1);
      if (lane == 0) {
        lst_n[qi] = cnt;
        lst_t[qi] = cnt < km ? -INFINITY : thr;
      }
    }
    __syncthreads();   // sc (aliasing ks) is read above; the next staging overwrites it
  }
  for (int jq = 0; jq < 16; ++jq) {
    const int qi = wave * 16 + jq;
    if (qi >= nq) break;
    const int own = (int)((q_pos0 + q0 + qi) / B);
    const int cnt = km > 0 ? lst_n[qi] : 0;
    const int lb = (lane < cnt) ? lst_b[qi][lane] : INT32_MAX;
    write_row(sel + (q0 + qi) * topk, topk, cnt, lb, own, window_first(own, win));
    if (sel_g)
      write_row(sel_g + (tab.q_row0[sq] + q0 + qi) * topk, topk, cnt,
                lane < cnt ? lb + tab.blk0[sq] : INT32_MAX, own + tab.blk0[sq],
                window_first(own, win) + tab.blk0[sq]);
  }
}

// ---------------------------------------------------------------------------
// Prefill, d_idx <= DW (DW = 64 or 128): the same tiles, lists and merge as
// topk_prefill_kernel, with the operands laid out for fewer memory steps.
// The dot product runs over DW/2 matrix-core steps, step t taking index
// columns t (lanes 0-31) and t + DW/2 (lanes 32-63) -- a sum over all
// columns in another order, which the near-tie bound covers.  So each lane's
// query operands are DW/2 consecutive columns of one query row, held in
// registers for the whole tile, and its summary operands four steps at a
// time are one 16-byte LDS read.  The next chunk of summaries is loaded
// into registers while the current chunk's products run, then written to
// LDS after the barrier that ends the current chunk's reads.  Columns past
// d_idx and rows past the chunk are zero.  VEC: d_idx is a multiple of 4 and
// both matrices 16-byte aligned (every row then is), so each summary piece
// is one unconditional 16-byte load from a valid address, zeroed after.
// ---------------------------------------------------------------------------
template <int KMAX, int DW, bool VEC>
__global__ __launch_bounds__(256) void topk_prefill_reg(
    const float *__restrict__ idx_q_all, SeqTab tab, const float *__restrict__ kmax_all,
    int d_idx, int topk, int win, int32_t *__restrict__ sel_all,
    int32_t *__restrict__ sel_g) {
  constexpr int kHalf = DW / 2;        // matrix-core steps; also columns per half-wave
  constexpr int kStr = DW + 4;         // LDS row stride (floats): 16-byte aligned rows
  constexpr int kV = DW / 4;           // float4 per row
  constexpr int kLd = kCB * kV / 256;  // float4 per thread per chunk
  __shared__ __attribute__((aligned(16))) float ks[kCB * kStr];
  __shared__ float sc[kQT][kCB + 1];
  __shared__ float lst_s[kQT][KMAX];
  __shared__ int lst_b[kQT][KMAX];
  __shared__ int lst_n[kQT];
  __shared__ float lst_t[kQT];   // entry threshold: the (K-1)-th score, -inf until full
  __shared__ int lst_lim[kQT];   // first block past the query's candidates (< 2^31)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Heavier (later) tiles first.
  const int64_t tile_g = (int64_t)tab.qt0[tab.n] - 1 - blockIdx.x;
  const int sq = prefix_find(tab.qt0, tab.n, tile_g);
  const int64_t tile = tile_g - tab.qt0[sq];
  const int64_t n_q = seq_nq(tab, sq), q_pos0 = tab.q_pos0[sq];
  const int B = tab.B;
  const float *idx_q = idx_q_all + tab.q_row0[sq] * d_idx;
  const float *kmax = kmax_all + (int64_t)tab.blk0[sq] * d_idx;
  int32_t *sel = sel_all + tab.q_row0[sq] * topk;
  const int64_t q0 = tile * kQT;
  const int nq = (int)(n_q - q0 < kQT ? n_q - q0 : kQT);
  const int km = topk - win;   // picks by score; the window win is forced
  const int64_t cand_last = (q_pos0 + q0 + nq - 1) / B - win + 1;
  const bool vq = (d_idx & 3) == 0 && (reinterpret_cast<uintptr_t>(idx_q) & 15) == 0;
  const bool vk = (d_idx & 3) == 0 && (reinterpret_cast<uintptr_t>(kmax) & 15) == 0;

  // four consecutive columns c .. c+3 of row r of a [*, d_idx] matrix (zero
  // past d_idx), with one 16-byte load when rows are aligned
  auto load4 = [&](const float *m, bool vec, int64_t r, int c) {
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (vec) {
      if (c < d_idx) x = *reinterpret_cast<const float4 *>(m + r * d_idx + c);
    } else {
      const float *p = m + r * d_idx;
      if (c < d_idx) x.x = p[c];
      if (c + 1 < d_idx) x.y = p[c + 1];
      if (c + 2 < d_idx) x.z = p[c + 2];
      if (c + 3 < d_idx) x.w = p[c + 3];
    }
    return x;
  };

  const int qw = wave >> 1, bw = wave & 1;
  const int h = lane >> 5, j = lane & 31;
  // this lane's query operands: row 32*qw + j, columns kHalf*h .. + kHalf-1
  float qreg[kHalf];
  {
    const int qr = 32 * qw + j;
#pragma unroll
    for (int u = 0; u < kHalf / 4; ++u) {
      const float4 x = qr < nq ? load4(idx_q, vq, q0 + qr, kHalf * h + 4 * u)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
      qreg[4 * u] = x.x;
      qreg[4 * u + 1] = x.y;
      qreg[4 * u + 2] = x.z;
      qreg[4 * u + 3] = x.w;
    }
  }
  // the next chunk's summaries, in flight in registers (b0 < cand_last:
  // row b0 exists)
  float4 kn[kLd];
  auto fetch = [&](int64_t b0) {
    const int nbk = (int)(cand_last - b0 < kCB ? cand_last - b0 : kCB);
#pragma unroll
    for (int i = 0; i < kLd; ++i) {
      const int e = tid + 256 * i, r = e / kV, c = 4 * (e % kV);
      if constexpr (VEC) {
        const bool ok = r < nbk && c < d_idx;
        const float4 x = *reinterpret_cast<const float4 *>(
            kmax + (b0 + (ok ? r : 0)) * d_idx + (ok ? c : 0));
        kn[i] = ok ? x : make_float4(0.f, 0.f, 0.f, 0.f);
      } else {
        kn[i] = r < nbk ? load4(kmax, vk, b0 + r, c) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  auto put = [&]() {
#pragma unroll
    for (int i = 0; i < kLd; ++i) {
      const int e = tid + 256 * i, r = e / kV, c = 4 * (e % kV);
      *reinterpret_cast<float4 *>(&ks[r * kStr + c]) = kn[i];
    }
  };

  if (tid < kQT) {
    lst_n[tid] = 0;
    lst_t[tid] = -INFINITY;
    // one 64-bit division per query, not one per query and chunk
    const int64_t lim = (q_pos0 + q0 + tid) / B - win + 1;
    lst_lim[tid] = (int)(lim < INT32_MAX ? lim : INT32_MAX);
  }
  for (int e = tid; e < kQT * KMAX; e += 256) {
    lst_s[e / KMAX][e % KMAX] = -INFINITY;
    lst_b[e / KMAX][e % KMAX] = -1;
  }
  if (km > 0 && cand_last > 0) {
    fetch(0);
    put();
  }
  __syncthreads();

  for (int64_t b0 = 0; km > 0 && b0 < cand_last; b0 += kCB) {
    const int nbk = (int)(cand_last - b0 < kCB ? cand_last - b0 : kCB);
    const bool more = b0 + kCB < cand_last;
    if (more) fetch(b0 + kCB);   // lands under this chunk's products
    f32x16s d;
#pragma unroll
    for (int r = 0; r < 16; ++r) d[r] = 0.f;
    const float *krow = &ks[(32 * bw + j) * kStr + kHalf * h];
#pragma unroll
    for (int u = 0; u < kHalf / 4; ++u) {
      const float4 kv = *reinterpret_cast<const float4 *>(krow + 4 * u);
      d = __builtin_amdgcn_mfma_f32_32x32x2f32(qreg[4 * u], kv.x, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_32x32x2f32(qreg[4 * u + 1], kv.y, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_32x32x2f32(qreg[4 * u + 2], kv.z, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_32x32x2f32(qreg[4 * u + 3], kv.w, d, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[32 * qw + 8 * (r >> 2) + 4 * h + (r & 3)][32 * bw + j] = d[r];
    __syncthreads();   // scores visible; every wave done reading ks
    if (more) put();   // the next chunk, for after the merge
    // Merge: wave w owns queries 16w .. 16w+15.  Query jq's candidate mask
    // (a wave ballot) is kept in lane jq of (mlo, mhi), where each insertion
    // group fetches its own with a cross-lane read.
    uint32_t need = 0;
    int mlo = 0, mhi = 0;
#pragma unroll
    for (int jq = 0; jq < 16; ++jq) {
      const int qi = wave * 16 + jq;
      const int lrel = lst_lim[qi] - (int)b0;   // b0 < cand_last < 2^31
      const float sv = sc[qi][lane];
      const float t = lst_t[qi];
      const bool valid = qi < nq && lane < nbk && lane < lrel;
      const uint64_t m = __ballot(valid && sv > t);
      mlo = lane == jq ? (int)(uint32_t)m : mlo;
      mhi = lane == jq ? (int)(uint32_t)(m >> 32) : mhi;
      if (m) need |= 1u << jq;
    }
    // Insertions, several queries at once: the wave splits into groups of
    // S lanes (S >= km), group gr holding the list of one query (entry gl in
    // lane gl of the group) and inserting that query's candidates in block
    // order, one per pass -- the same sequence of insertions as one query at
    // a time, so the same lists.
    {
      const int S = km <= 8 ? 8 : (km <= 16 ? 16 : (km <= 32 ? 32 : 64));
      const int NG = 64 / S;
      const int gr = lane / S, gl = lane % S;
      const uint64_t gmask = S == 64 ? ~0ull : ((1ull << S) - 1) << (gr * S);
      for (int r0 = 0; r0 < 16; r0 += NG) {
        if (!((need >> r0) & ((1u << NG) - 1))) continue;
        const int jq = r0 + gr;
        const int qi = wave * 16 + jq;
        uint64_t mask = ((uint64_t)(uint32_t)__shfl(mhi, jq, 64) << 32) |
                        (uint64_t)(uint32_t)__shfl(mlo, jq, 64);
        int cnt = lst_n[qi];
        float ls = gl < km ? lst_s[qi][gl] : -INFINITY;
        int lb = gl < km ? lst_b[qi][gl] : -1;
        float thr = lst_t[qi];
        // each pass reads the score of the group's next candidate ahead, so
        // the LDS round trip overlaps the current insertion
        int nsrc = mask != 0 ? __ffsll((unsigned long long)mask) - 1 : 0;
        float nsj = sc[qi][nsrc];
        while (__ballot(mask != 0)) {
          const bool act = mask != 0;
          const int src = nsrc;
          const float sj = nsj;
          if (act) mask &= mask - 1;
          nsrc = mask != 0 ? __ffsll((unsigned long long)mask) - 1 : 0;
          nsj = sc[qi][nsrc];
          // rank among the group's entries; below km it enters (a full list:
          // strictly above the km-th entry, which a tie does not pass)
          const int pos = __popcll(__ballot(gl < cnt && ls >= sj) & gmask);
          const bool ins = act && pos < km;
          // entries shift down one lane (DPP; a group's first lane never takes
          // its neighbour's value: pos >= 0)
          const float up_s = prev_lane_f(ls);
          const int up_b = prev_lane_i(lb);
          const int last = cnt < km - 1 ? cnt : km - 1;
          if (ins && gl > pos && gl <= last) {
            ls = up_s;
            lb = up_b;
          }
          if (ins && gl == pos) {
            ls = sj;
            lb = (int)b0 + src;
          }
          if (ins) cnt = cnt + 1 < km ? cnt + 1 : km;
        }
        const float kth = __shfl(ls, gr * S + km - 1);
        thr = cnt < km ? -INFINITY : kth;
        if (gl < km) {
          lst_s[qi][gl] = ls;
          lst_b[qi][gl] = lb;
        }
        if (gl == 0) {
          lst_n[qi] = cnt;
          lst_t[qi] = thr;
        }
      }
    }
    __syncthreads();   // sc read above and ks written: the next chunk may start
  }
  for (int jq = 0; jq < 16; ++jq) {
    const int qi = wave * 16 + jq;
    if (qi >= nq) break;
    const int own = (int)((q_pos0 + q0 + qi) / B);
    const int cnt = km > 0 ? lst_n[qi] : 0;
    const int lb = (lane < cnt) ? lst_b[qi][lane] : INT32_MAX;
    write_row(sel + (q0 + qi) * topk, topk, cnt, lb, own, window_first(own, win));
    if (sel_g)
      write_row(sel_g + (tab.q_row0[sq] + q0 + qi) * topk, topk, cnt,
                lane < cnt ? lb + tab.blk0[sq] : INT32_MAX, own + tab.blk0[sq],
                window_first(own, win) + tab.blk0[sq]);
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
__global__ __launch_bounds__(256) void topk_decode_kernel(
    const float *__restrict__ idx_q, const int64_t *__restrict__ seq_len,
    const float *__restrict__ kmax, int64_t nb_max, int d_idx, int B, int km, int win,
    float *__restrict__ ws_s, int *__restrict__ ws_b, int n_chunks) {
  const int s = blockIdx.y;
  const int64_t len = seq_len[s];
  const int64_t own = len >= 1 ? (len - 1) / B : 0;   // the query sits at len - 1
  decode_scan_chunk(idx_q + (int64_t)s * d_idx, kmax + (int64_t)s * nb_max * d_idx,
                    own - win + 1, nb_max, d_idx, km, blockIdx.x,
                    ws_s + ((int64_t)s * n_chunks + blockIdx.x) * km,
                    ws_b + ((int64_t)s * n_chunks + blockIdx.x) * km);
}

__global__ __launch_bounds__(64) void topk_decode_merge(
    const int64_t *__restrict__ seq_len, int B, int topk, int win,
    const float *__restrict__ ws_s, const int *__restrict__ ws_b, int n_chunks,
    int32_t *__restrict__ sel) {
  __shared__ float st_s[2048];
  __shared__ int st_b[2048];
  const int s = blockIdx.x;
  const int64_t len = seq_len[s];
  const int km = topk - win;
  decode_merge_lists(ws_s + (int64_t)s * n_chunks * km, ws_b + (int64_t)s * n_chunks * km,
                     n_chunks, topk, win,
                     [&] { return (int)(len >= 1 ? (len - 1) / B : 0); },
                     sel + (int64_t)s * topk, st_s, st_b, 2048);
}

// A batch of queries of several sequences, each at its own position: query
// i of sequence q_seq[i] at q_pos[i] is scanned like a decode query (chunks
// of 64 blocks of its sequence's summaries, then the chunk lists merged).  A
// query whose sequence or position is out of range gets no candidates and a
// row of -1.
__device__ __forceinline__ bool batch_query_ok(int32_t s, int64_t p, int32_t n_seq,
                                               int64_t nb_max, int B) {
  return s >= 0 && s < n_seq && p >= 0 && p < nb_max * B;
}

__global__ __launch_bounds__(256) void topk_batch_kernel(
    const float *__restrict__ idx_q, const int32_t *__restrict__ q_seq,
    const int64_t *__restrict__ q_pos, const float *__restrict__ kmax, int32_t n_seq,
    int64_t nb_max, int d_idx, int B, int km, float *__restrict__ ws_s,
    int *__restrict__ ws_b, int n_chunks) {
  const int64_t i = blockIdx.x;
  const int32_t s = q_seq[i];
  const int64_t p = q_pos[i];
  const bool ok = batch_query_ok(s, p, n_seq, nb_max, B);
  const int64_t own = ok ? p / B : 0;
  float *out_s = ws_s + (i * n_chunks + blockIdx.y) * km;
  int *out_b = ws_b + (i * n_chunks + blockIdx.y) * km;
  if ((int64_t)blockIdx.y * kDecChunk >= own) {   // no candidate here (uniform): empty list
    for (int r = threadIdx.x; r < km; r += 256) {
      out_s[r] = -INFINITY;
      out_b[r] = -1;
    }
    return;
  }
  decode_scan_chunk(idx_q + i * d_idx, kmax + (int64_t)(ok ? s : 0) * nb_max * d_idx, own,
                    nb_max, d_idx, km, blockIdx.y, out_s, out_b);
}

__global__ __launch_bounds__(64) void topk_batch_merge(
    const int32_t *__restrict__ q_seq, const int64_t *__restrict__ q_pos, int32_t n_seq,
    int64_t nb_max, int B, int topk, const float *__restrict__ ws_s,
    const int *__restrict__ ws_b, int n_chunks, int32_t *__restrict__ sel) {
  __shared__ float st_s[2048];
  __shared__ int st_b[2048];
  const int64_t i = blockIdx.x;
  const int32_t s = q_seq[i];
  const int64_t p = q_pos[i];
  if (!batch_query_ok(s, p, n_seq, nb_max, B)) {   // uniform: one query per workgroup
    for (int k = threadIdx.x; k < topk; k += 64) sel[i * topk + k] = -1;
    return;
  }
  const int km = topk - 1;
  decode_merge_lists(ws_s + i * n_chunks * km, ws_b + i * n_chunks * km, n_chunks, topk, 1,
                     [&] { return (int)(p / B); }, sel + i * topk, st_s, st_b, 2048);
}

}  // namespace

hipError_t launch_topk_tab(const float *idx_q, const SeqTab &tab, const float *kmax,
                           int32_t d_idx, int32_t topk, int32_t win, int32_t *sel,
                           int32_t *sel_g, hipStream_t st) {
  const int64_t n_tiles = tab.qt0[tab.n];
  if (n_tiles <= 0) return hipSuccess;
  const dim3 grid((unsigned)n_tiles), wg(256);
  const bool full = d_idx <= kDFull;
#define MSA_TK(KM, FU)                                                                     \
  hipLaunchKernelGGL((topk_prefill_kernel<KM, FU>), grid, wg, 0, st, idx_q, tab, kmax, d_idx, \
                     topk, win, sel, sel_g)
  const bool vec = (d_idx & 3) == 0 && (reinterpret_cast<uintptr_t>(idx_q) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(kmax) & 15) == 0;
#define MSA_TR(KM, DW)                                                                       \
  do {                                                                                       \
    if (vec)                                                                                 \
      hipLaunchKernelGGL((topk_prefill_reg<KM, DW, true>), grid, wg, 0, st, idx_q, tab, kmax, \
                         d_idx, topk, win, sel, sel_g);                                      \
    else                                                                                     \
      hipLaunchKernelGGL((topk_prefill_reg<KM, DW, false>), grid, wg, 0, st, idx_q, tab,     \
                         kmax, d_idx, topk, win, sel, sel_g);                                \
  } while (0)
  if (d_idx <= 128) {   // query operands in registers
    if (topk - win <= 16) {
      if (d_idx <= 64)
        MSA_TR(16, 64);
      else
        MSA_TR(16, 128);
    } else {
      if (d_idx <= 64)
        MSA_TR(64, 64);
      else
        MSA_TR(64, 128);
    }
#undef MSA_TR
    return hipGetLastError();
  }
  if (topk - win <= 16) {
    if (full)
      MSA_TK(16, true);
    else
      MSA_TK(16, false);
  } else {
    if (full)
      MSA_TK(64, true);
    else
      MSA_TK(64, false);
  }
#undef MSA_TK
  return hipGetLastError();
}

hipError_t launch_topk_prefill(const float *idx_q, int64_t n_q, int64_t q_pos0,
                               const float *kmax, int64_t nb, int32_t d_idx,
                               int32_t block, int32_t topk, int32_t win, int32_t *sel,
                               hipStream_t st) {
  (void)nb;
  return launch_topk_tab(idx_q, seqtab_one(q_pos0, n_q, block), kmax, d_idx, topk, win, sel,
                         nullptr, st);
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
                              int32_t topk, int32_t win, int32_t *sel, void *ws,
                              hipStream_t st) {
  const int n_chunks = (int)((nb_max + kDecChunk - 1) / kDecChunk);
  const size_t n = (size_t)n_seq * n_chunks * (topk > 1 ? topk - 1 : 1);
  char *w = static_cast<char *>(ws);
  float *ws_s = reinterpret_cast<float *>(w);
  w += align256(n * sizeof(float));
  int *ws_b = reinterpret_cast<int *>(w);
  if (topk > win) {
    hipLaunchKernelGGL(topk_decode_kernel, dim3(n_chunks, n_seq), dim3(256), 0, st,
                       idx_q, seq_len, kmax, nb_max, d_idx, block, topk - win, win, ws_s,
                       ws_b, n_chunks);
  }
  hipLaunchKernelGGL(topk_decode_merge, dim3(n_seq), dim3(64), 0, st, seq_len,
                     block, topk, win, ws_s, ws_b, n_chunks, sel);
  return hipGetLastError();
}

// Layout as the decode selection's: [chunk scores][chunk block ids] per query.
size_t topk_batch_ws_bytes(int64_t n_q, int64_t nb_max, int32_t topk) {
  const int64_t n_chunks = (nb_max + kDecChunk - 1) / kDecChunk;
  const size_t n = (size_t)n_q * n_chunks * (topk > 1 ? topk - 1 : 1);
  return align256(n * sizeof(float)) + align256(n * sizeof(int));
}

hipError_t launch_topk_batch(const float *idx_q, int64_t n_q, const int32_t *q_seq,
                             const int64_t *q_pos, const float *kmax, int32_t n_seq,
                             int64_t nb_max, int32_t d_idx, int32_t block, int32_t topk,
                             int32_t *sel, void *ws, hipStream_t st) {
  if (n_q <= 0) return hipSuccess;
  const int n_chunks = (int)((nb_max + kDecChunk - 1) / kDecChunk);
  const size_t n = (size_t)n_q * n_chunks * (topk > 1 ? topk - 1 : 1);
  char *w = static_cast<char *>(ws);
  float *ws_s = reinterpret_cast<float *>(w);
  w += align256(n * sizeof(float));
  int *ws_b = reinterpret_cast<int *>(w);
  if (topk > 1)
    hipLaunchKernelGGL(topk_batch_kernel, dim3((unsigned)n_q, n_chunks), dim3(256), 0, st,
                       idx_q, q_seq, q_pos, kmax, n_seq, nb_max, d_idx, block, topk - 1, ws_s,
                       ws_b, n_chunks);
  hipLaunchKernelGGL(topk_batch_merge, dim3((unsigned)n_q), dim3(64), 0, st, q_seq, q_pos,
                     n_seq, nb_max, block, topk, ws_s, ws_b, n_chunks, sel);
  return hipGetLastError();
}

}  // namespace msa
