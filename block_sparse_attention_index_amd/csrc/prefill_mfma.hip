// prefill_mfma.hip -- sparse-branch prefill on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16), d = 128.  Same two-pass KV-outer organisation
// as the VALU kernels in prefill.hip (sparse branch of "MiniMax M3模型算力成本
// 大幅降低原因深度解析"; section 2.2 "KV Outer Gather Q：MSA 的关键设计" of
// chenxutan.com's "MiniMax M3 深度实战"):
//   pass A  one workgroup per (KV block b, KV head g, tile of 256/G queries
//           from row b's non-own list): K[g,b] and V[g,b] are staged through
//           LDS in 64-key chunks and applied to all 256 gathered query rows
//           (tile tokens x the G query heads of group g);
//   pass B  one workgroup per (block b, head g, tile of b's own tokens):
//           causal attention inside the own block, then the log-sum-exp merge
//           with pass A's partials; writes O and LSE.
//
// Each wave owns 64 query rows as two 32-row N-blocks.  Scores are computed
// transposed, S^T = K Q^T (keys = MFMA rows), so a lane holds 16 keys of ONE
// query row: the row max needs a single exchange with lane l^32 and the
// softmax statistics stay per lane.  P^T leaves the accumulator already in
// the B-operand layout of O^T = V^T P^T, provided V^T's k-slots use the same
// key order; V is therefore staged transposed in LDS.  Lazy rescaling: the
// running reference max moves only when a row's max exceeds it by more than
// 8 (so every weight is at most 2^8), which removes most O rescales.
#include "msa_internal.h"
#include "prefill_common.h"

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;          // head dim handled here
constexpr int kKC = 64;          // keys per staged chunk
constexpr int kKStr = kD + 8;    // K row stride in LDS, bf16 elements (272 B)
constexpr int kVStr = kKC + 4;   // V^T row stride in LDS, bf16 elements (136 B)
constexpr float kLazy = 8.f;     // reference-max slack (log2 units)

struct MfmaSmem {
  uint16_t Ks[kKC * kKStr];
  uint16_t Vt[kD * kVStr];
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Stage keys [row0, row0+nrows) of one (head, block) slice: K row-major with
// padded rows, V transposed (V^T[c][key]).  Rows past nrows are zero.
__device__ __forceinline__ void stage(MfmaSmem &sm, const uint16_t *k,
                                      const uint16_t *v, int64_t row0,
                                      int nrows) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < (kKC * kD / 8) / 256; ++it) {
    const int x = tid + 256 * it;
    const int key = x >> 4, seg = x & 15;
    u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (key < nrows) {
      kv = *reinterpret_cast<const u32x4 *>(k + (row0 + key) * kD + seg * 8);
      vv = *reinterpret_cast<const u32x4 *>(v + (row0 + key) * kD + seg * 8);
    }
    *reinterpret_cast<u32x4 *>(&sm.Ks[key * kKStr + seg * 8]) = kv;
    const uint16_t *ve = reinterpret_cast<const uint16_t *>(&vv);
#pragma unroll
    for (int i = 0; i < 8; ++i) sm.Vt[(seg * 8 + i) * kVStr + key] = ve[i];
  }
}

template <int G, bool OWN>
__global__ __launch_bounds__(256, 1) void prefill_mfma_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, int64_t kv_stride, int64_t q_pos0,
    int64_t n_q, int hq, int B, const int32_t *__restrict__ row_ptr,
    const int32_t *__restrict__ q_list, const int32_t *__restrict__ tile_ptr,
    int64_t nb, const int32_t *__restrict__ sel, int topk,
    const int32_t *__restrict__ slot, float scale_log2,
    float *__restrict__ part_o, float *__restrict__ part_lse, int64_t n_part,
    float *__restrict__ o, float *__restrict__ lse) {
  constexpr int TPN = 32 / G;    // tokens per 32-row N-block
  constexpr int TPW = 2 * TPN;   // tokens per wave
  constexpr int TPT = 4 * TPW;   // tokens per tile (workgroup)
  __shared__ MfmaSmem sm;

  const int g = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = lane >> 5, j = lane & 31;

  // ---- the tile: block b, its key count, and each N-block row's query ----
  int64_t b, nkeys, e0 = 0, e_end = 0, tok0 = 0, min_pos;
  if constexpr (!OWN) {
    const int64_t w = blockIdx.x;
    if (w >= tile_ptr[nb]) return;
    b = find_row(tile_ptr, nb, w);
    const int64_t own_b =
        own_through(b, q_pos0, n_q, B) - own_through(b - 1, q_pos0, n_q, B);
    e0 = row_ptr[b] + own_b + (w - tile_ptr[b]) * TPT;
    e_end = row_ptr[b + 1];
    nkeys = B;
    if (b * B + nkeys > kv_stride) nkeys = kv_stride - b * B;  // invalid input only
    min_pos = INT64_MAX;
  } else {
    const int tpb = (B + TPT - 1) / TPT;
    b = q_pos0 / B + blockIdx.x / tpb;
    tok0 = b * B + (int64_t)(blockIdx.x % tpb) * TPT;
    int64_t hi = tok0 + TPT - 1;
    if (hi > b * B + B - 1) hi = b * B + B - 1;
    if (hi > q_pos0 + n_q - 1) hi = q_pos0 + n_q - 1;
    if (hi < tok0 || hi < q_pos0) return;
    nkeys = hi - b * B + 1;
    min_pos = tok0;
  }

  int64_t qi[2], pos[2];
  bool act[2];
  int head[2];
  bf16x8 qf[2][8];
#pragma unroll
  for (int nbk = 0; nbk < 2; ++nbk) {
    const int tl = wave * TPW + nbk * TPN + j / G;
    head[nbk] = j % G;
    if constexpr (!OWN) {
      const int64_t e = e0 + tl;
      int64_t x = e < e_end ? q_list[e] : -1;
      act[nbk] = x >= 0 && x < n_q;
      qi[nbk] = act[nbk] ? x : 0;
      pos[nbk] = q_pos0 + qi[nbk];
    } else {
      const int64_t p = tok0 + tl;
      act[nbk] = p >= q_pos0 && p < q_pos0 + n_q && p < b * B + B;
      pos[nbk] = p < b * B + B ? p : b * B + B - 1;
      qi[nbk] = act[nbk] ? p - q_pos0 : 0;
    }
    const uint16_t *qp = q + ((qi[nbk] * hq + (int64_t)g * G + head[nbk]) * kD);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (act[nbk]) x = *reinterpret_cast<const u32x4 *>(qp + cc * 16 + 8 * h);
      qf[nbk][cc] = as_bf16x8(x);
    }
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int nbk = 0; nbk < 2; ++nbk)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nbk][cb][r] = 0.f;
  float mref[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};

  const uint16_t *kb = k + ((int64_t)g * kv_stride) * kD;
  const uint16_t *vb = v + ((int64_t)g * kv_stride) * kD;
  for (int64_t kc = 0; kc < nkeys; kc += kKC) {
    const int nrows = (int)(nkeys - kc < kKC ? nkeys - kc : kKC);
    __syncthreads();
    stage(sm, kb, vb, b * B + kc, nrows);
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int koff0 = (int)kc + sub * 32;          // key offset in block
      if (koff0 >= nkeys) break;
      f32x16 s[2];
#pragma unroll
      for (int nbk = 0; nbk < 2; ++nbk)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nbk][r] = 0.f;
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const u32x4 kraw = *reinterpret_cast<const u32x4 *>(
            &sm.Ks[(sub * 32 + j) * kKStr + cc * 16 + 8 * h]);
        const bf16x8 kf = as_bf16x8(kraw);
        s[0] = mfma32(kf, qf[0][cc], s[0]);
        s[1] = mfma32(kf, qf[1][cc], s[1]);
      }
      const bool need_mask =
          koff0 + 31 >= nkeys || (OWN && b * B + koff0 + 31 > min_pos);
      bf16x8 pb[2][2];
#pragma unroll
      for (int nbk = 0; nbk < 2; ++nbk) {
        if (need_mask) {
          const int64_t lim = OWN ? pos[nbk] - b * B : nkeys - 1;
          const int64_t lim2 = lim < nkeys - 1 ? lim : nkeys - 1;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int koff = koff0 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (koff > lim2) s[nbk][r] = -INFINITY;
          }
        }
        float mloc = s[nbk][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mloc = fmaxf(mloc, s[nbk][r]);
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        const float mt = mloc * scale_log2;
        if (__ballot(mt > mref[nbk] + kLazy)) {
          const float mnew = fmaxf(mref[nbk], mt);
          const float alpha = fast_exp2(mref[nbk] - mnew);
          lsum[nbk] *= alpha;
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[nbk][cb][r] *= alpha;
          mref[nbk] = mnew;
        }
        const float mr = mref[nbk];
        f32x8 p0, p1;
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          p0[r] = fast_exp2(fmaf(s[nbk][r], scale_log2, -mr));
          p1[r] = fast_exp2(fmaf(s[nbk][r + 8], scale_log2, -mr));
          ps += p0[r] + p1[r];
        }
        lsum[nbk] += ps;
        pb[nbk][0] = __builtin_convertvector(p0, bf16x8);
        pb[nbk][1] = __builtin_convertvector(p1, bf16x8);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const uint16_t *vr = &sm.Vt[(cb * 32 + j) * kVStr + sub * 32 + 16 * ks + 4 * h];
          const u32x2 lo = *reinterpret_cast<const u32x2 *>(vr);
          const u32x2 hi = *reinterpret_cast<const u32x2 *>(vr + 8);
          const u32x4 vraw = {lo[0], lo[1], hi[0], hi[1]};
          const bf16x8 vf = as_bf16x8(vraw);
          acc[0][cb] = mfma32(vf, pb[0][ks], acc[0][cb]);
          acc[1][cb] = mfma32(vf, pb[1][ks], acc[1][cb]);
        }
      }
    }
  }

  // ---- epilogue ----
#pragma unroll
  for (int nbk = 0; nbk < 2; ++nbk) {
    const float ltot = lsum[nbk] + __shfl_xor(lsum[nbk], 32, 64);
    const int hh = g * G + head[nbk];
    if constexpr (!OWN) {
      if (!act[nbk]) continue;
      const int64_t e = e0 + wave * TPW + nbk * TPN + j / G;
      const int64_t n_idx = e - own_through(b, q_pos0, n_q, B);
      if (n_idx < 0 || n_idx >= n_part) continue;
      const float inv = 1.f / ltot;
      float *dst = part_o + (n_idx * hq + hh) * (int64_t)kD;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          float4 val = make_float4(acc[nbk][cb][4 * rg] * inv, acc[nbk][cb][4 * rg + 1] * inv,
                                   acc[nbk][cb][4 * rg + 2] * inv, acc[nbk][cb][4 * rg + 3] * inv);
          *reinterpret_cast<float4 *>(dst + cb * 32 + 8 * rg + 4 * h) = val;
        }
      if (h == 0) part_lse[n_idx * hq + hh] = mref[nbk] + __log2f(ltot);
    } else {
      if (!act[nbk]) continue;
      const int64_t i = qi[nbk];
      const int32_t *srow = sel + i * topk;
      const int32_t *xrow = slot + i * topk;
      const float own2 = mref[nbk] + __log2f(ltot);
      float mx = own2;
      for (int kk = 0; kk < topk; ++kk) {
        const int32_t bk = srow[kk];
        if (bk < 0 || bk >= b) continue;
        const int64_t n_idx = xrow[kk] - own_through(bk, q_pos0, n_q, B);
        if (n_idx < 0 || n_idx >= n_part) continue;
        mx = fmaxf(mx, part_lse[n_idx * hq + hh]);
      }
      float z = fast_exp2(own2 - mx);
      const float wo = z / ltot;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nbk][cb][r] *= wo;
      for (int kk = 0; kk < topk; ++kk) {
        const int32_t bk = srow[kk];
        if (bk < 0 || bk >= b) continue;
        const int64_t n_idx = xrow[kk] - own_through(bk, q_pos0, n_q, B);
        if (n_idx < 0 || n_idx >= n_part) continue;
        const float wk = fast_exp2(part_lse[n_idx * hq + hh] - mx);
        z += wk;
        const float *src = part_o + (n_idx * hq + hh) * (int64_t)kD;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const float4 pv = *reinterpret_cast<const float4 *>(src + cb * 32 + 8 * rg + 4 * h);
            acc[nbk][cb][4 * rg] = fmaf(wk, pv.x, acc[nbk][cb][4 * rg]);
            acc[nbk][cb][4 * rg + 1] = fmaf(wk, pv.y, acc[nbk][cb][4 * rg + 1]);
            acc[nbk][cb][4 * rg + 2] = fmaf(wk, pv.z, acc[nbk][cb][4 * rg + 2]);
            acc[nbk][cb][4 * rg + 3] = fmaf(wk, pv.w, acc[nbk][cb][4 * rg + 3]);
          }
      }
      const float invz = 1.f / z;
      float *dst = o + (i * hq + hh) * (int64_t)kD;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          float4 val = make_float4(acc[nbk][cb][4 * rg] * invz, acc[nbk][cb][4 * rg + 1] * invz,
                                   acc[nbk][cb][4 * rg + 2] * invz, acc[nbk][cb][4 * rg + 3] * invz);
          *reinterpret_cast<float4 *>(dst + cb * 32 + 8 * rg + 4 * h) = val;
        }
      if (lse && h == 0) lse[i * hq + hh] = (mx + __log2f(z)) * kLn2;
    }
  }
}

template <int G>
hipError_t launch_mfma_g(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         int64_t kv_stride, int64_t q_pos0, int64_t n_q, int hq,
                         int hkv, int B, const int32_t *sel, int topk,
                         const int32_t *row_ptr, const int32_t *q_list,
                         const int32_t *slot, float scale, float *o, float *lse,
                         int32_t *tile_ptr, float *part_o, float *part_lse,
                         int64_t n_part, hipStream_t st) {
  constexpr int TPT = 256 / G;
  const int64_t nb = (q_pos0 + n_q + B - 1) / B;
  const float sl2 = scale * kLog2e;
  if (n_part > 0) {
    hipLaunchKernelGGL(prefill_tiles, dim3(1), dim3(1024), 0, st, row_ptr, nb,
                       q_pos0, n_q, B, TPT, tile_ptr);
    const int64_t grid = n_part / TPT + nb;
    hipLaunchKernelGGL((prefill_mfma_kernel<G, false>), dim3((unsigned)grid, hkv),
                       dim3(256), 0, st, q, k, v, kv_stride, q_pos0, n_q, hq, B,
                       row_ptr, q_list, tile_ptr, nb, sel, topk, slot, sl2, part_o,
                       part_lse, n_part, o, lse);
  }
  const int64_t b_first = q_pos0 / B, b_last = (q_pos0 + n_q - 1) / B;
  const int64_t tiles = (b_last - b_first + 1) * ((B + TPT - 1) / TPT);
  hipLaunchKernelGGL((prefill_mfma_kernel<G, true>), dim3((unsigned)tiles, hkv),
                     dim3(256), 0, st, q, k, v, kv_stride, q_pos0, n_q, hq, B,
                     row_ptr, q_list, tile_ptr, nb, sel, topk, slot, sl2, part_o,
                     part_lse, n_part, o, lse);
  return hipGetLastError();
}

}  // namespace

bool mfma_prefill_supported(int32_t dtype, int32_t d, int32_t group) {
  return dtype == 1 && d == kD &&
         (group == 1 || group == 2 || group == 4 || group == 8 || group == 16);
}

hipError_t launch_prefill_mfma(const void *q, const void *k, const void *v,
                               int64_t kv_stride, int64_t q_pos0, int64_t n_q,
                               int32_t hq, int32_t hkv, int32_t d,
                               int32_t block, const int32_t *sel, int32_t topk,
                               const int32_t *row_ptr, const int32_t *q_list,
                               const int32_t *slot, float scale, float *o,
                               float *lse, void *ws, hipStream_t st) {
  (void)d;
  const int G = hq / hkv;
  const int64_t nb = (q_pos0 + n_q + block - 1) / block;
  const int64_t np = nonown_pairs(q_pos0, n_q, block, topk);
  char *w = static_cast<char *>(ws);
  int32_t *tile_ptr = reinterpret_cast<int32_t *>(w);
  w += align256((size_t)(nb + 1) * 4);
  float *part_o = reinterpret_cast<float *>(w);
  w += align256((size_t)np * hq * d * 4);
  float *part_lse = reinterpret_cast<float *>(w);
  const uint16_t *qq = static_cast<const uint16_t *>(q);
  const uint16_t *kk = static_cast<const uint16_t *>(k);
  const uint16_t *vv = static_cast<const uint16_t *>(v);
#define MSA_MF(GG)                                                             \
  case GG:                                                                     \
    return launch_mfma_g<GG>(qq, kk, vv, kv_stride, q_pos0, n_q, hq, hkv,      \
                             block, sel, topk, row_ptr, q_list, slot, scale, o, \
                             lse, tile_ptr, part_o, part_lse, np, st);
  switch (G) {
    MSA_MF(1)
    MSA_MF(2)
    MSA_MF(4)
    MSA_MF(8)
    MSA_MF(16)
    default:
      break;
  }
#undef MSA_MF
  return hipErrorInvalidValue;
}

}  // namespace msa
