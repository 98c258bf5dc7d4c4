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
template <int KMAX, bool FULL>
__global__ __launch_bounds__(256) void topk_prefill_kernel(
    const float *__restrict__ idx_q, int64_t n_q, int64_t q_pos0,
    const float *__restrict__ kmax, int d_idx, int B, int topk, int win,
    int32_t *__restrict__ sel) {
  constexpr int kW = FULL ? kDFull : kDC;   // staged columns
  constexpr int kPad = kW + 1;
  __shared__ float qs[kQT][kPad];
  __shared__ float ks[kCB][kPad];
  __shared__ float lst_s[kQT][KMAX];
  __shared__ int lst_b[kQT][KMAX];
  __shared__ int lst_n[kQT];
  __shared__ float lst_t[kQT];   // entry threshold: the (K-1)-th score, -inf until full
  // scores alias the block rows (written after the MFMAs' last read of them,
  // read before the next chunk's staging; both sides fenced)
  float(*sc)[kPad] = ks;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Heavier (later) tiles first.
  const int64_t n_tiles = (n_q + kQT - 1) / kQT;
  const int64_t tile = n_tiles - 1 - blockIdx.x;
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
      const int64_t lim = (q_pos0 + q0 + qi) / B - win + 1;
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

}  // namespace

hipError_t launch_topk_prefill(const float *idx_q, int64_t n_q, int64_t q_pos0,
                               const float *kmax, int64_t nb, int32_t d_idx,
                               int32_t block, int32_t topk, int32_t win, int32_t *sel,
                               hipStream_t st) {
  (void)nb;
  const int64_t n_tiles = (n_q + kQT - 1) / kQT;
  const dim3 grid((unsigned)n_tiles), wg(256);
  const bool full = d_idx <= kDFull;
  if (topk - win <= 16) {
    if (full)
      hipLaunchKernelGGL((topk_prefill_kernel<16, true>), grid, wg, 0, st, idx_q, n_q,
                         q_pos0, kmax, d_idx, block, topk, win, sel);
    else
      hipLaunchKernelGGL((topk_prefill_kernel<16, false>), grid, wg, 0, st, idx_q, n_q,
                         q_pos0, kmax, d_idx, block, topk, win, sel);
  } else {
    if (full)
      hipLaunchKernelGGL((topk_prefill_kernel<64, true>), grid, wg, 0, st, idx_q, n_q,
                         q_pos0, kmax, d_idx, block, topk, win, sel);
    else
      hipLaunchKernelGGL((topk_prefill_kernel<64, false>), grid, wg, 0, st, idx_q, n_q,
                         q_pos0, kmax, d_idx, block, topk, win, sel);
  }
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

}  // namespace msa
