// decode.hip -- sparse-branch decode: one new query per sequence attends to
// its selected blocks (decode part of section 3.3 of chenxutan.com's "MiniMax
// M3 深度实战"; GQA over the chosen blocks only, sparse branch of "MiniMax M3
// 模型算力成本大幅降低原因深度解析").
//
// Split-KV.  Work item = (sequence s, KV head g, selected slot kk, chunk of up
// to 128 keys of that block), so even one sequence fills the chip.  The item
// stages its K and V rows in LDS once with 16-byte loads and writes a
// normalised partial output and its base-2 log-sum-exp for every query head
// of group g; a second kernel merges the partials of each (sequence, head) by
// log-sum-exp.  (A same-kernel merge by the last-arriving item was measured
// slower: the cross-XCD release fence it needs costs more than a launch.)
// bf16 with d = 128 computes each 32-key slice on the matrix cores -- S^T =
// K Q^T with the heads padded to 32 MFMA columns, O^T = V^T P^T with V^T read
// by ds_read_b64_tr_b16, as in the prefill kernel -- and combines its four
// waves through LDS; other shapes use a VALU kernel.  HBM-bound: K and V are
// read once.
#include "msa_internal.h"
#include "mfma_common.h"

namespace msa {
namespace {

constexpr int kDK = 128;   // keys per work item (at most)

template <typename T>
__device__ __forceinline__ float ldx(const T *p, int64_t i);
template <>
__device__ __forceinline__ float ldx<float>(const float *p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float ldx<uint16_t>(const uint16_t *p, int64_t i) {
  return bf16_to_f32(p[i]);
}

// Raw element stride of a staged row (padding keeps lane = key reads
// conflict-free) and element count of a 16-byte vector.
template <typename T, int D>
struct DecShape {
  static constexpr int kVec = 16 / (int)sizeof(T);
  static constexpr int kStr = D + kVec;
};

template <typename T, int D>
struct DecKV {
  T K[kDK * DecShape<T, D>::kStr];
  T V[kDK * DecShape<T, D>::kStr];
};

template <typename T, int G, int D>
struct DecSmem {
  union {
    DecKV<T, D> kv;
  } u;
  float Q[G][D];
  float P[kDK][G];            // softmax weights, heads of a key contiguous
};

// 8 consecutive staged elements of a row as floats (one 16-byte LDS read for
// bf16, two for fp32).
__device__ __forceinline__ void lds8(const uint16_t *p, float (&f)[8]) {
  const uint4 r = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void lds8(const float *p, float (&f)[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
__device__ __forceinline__ void lds2(const uint16_t *p, float &a, float &b) {
  const uint32_t w = *reinterpret_cast<const uint32_t *>(p);
  a = __uint_as_float(w << 16);
  b = __uint_as_float(w & 0xffff0000u);
}
__device__ __forceinline__ void lds2(const float *p, float &a, float &b) {
  const float2 v = *reinterpret_cast<const float2 *>(p);
  a = v.x;
  b = v.y;
}

// grid = (topk * nsub, Hkv, n_seq); nsub = ceil(B / 128)
template <typename T, int G, int D>
__global__ __launch_bounds__(256) void decode_attn(
    const T *__restrict__ q, const T *__restrict__ kc, const T *__restrict__ vc,
    int64_t len_max, const int64_t *__restrict__ seq_len, int hq, int B,
    const int32_t *__restrict__ sel, int topk, int nsub, float scale_log2,
    float *__restrict__ part_o, float *__restrict__ part_lse) {
  using S = DecShape<T, D>;
  constexpr int HPW = (G + 3) / 4;   // query heads per wave
  constexpr int CPL = D / 64;        // output columns per lane (consecutive)
  __shared__ DecSmem<T, G, D> sm;
  const int s = blockIdx.z, g = blockIdx.y;
  const int kk = blockIdx.x / nsub, sub = blockIdx.x % nsub;
  const int hkv = gridDim.y, np = gridDim.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h0 = wave * HPW;
  const int nh = h0 >= G ? 0 : (G - h0 < HPW ? G - h0 : HPW);

  int64_t len = seq_len[s];
  if (len > len_max) len = len_max;
  const int64_t pos = len - 1;
  const int32_t b = sel[(int64_t)s * topk + kk];
  const int64_t t0 = (int64_t)b * B + (int64_t)sub * kDK;
  int64_t nkeys = (b < 0 || len < 1) ? 0 : pos - t0 + 1;
  if (nkeys > kDK) nkeys = kDK;
  if (nkeys > B - sub * kDK) nkeys = B - sub * kDK;   // stay inside block b
  const int64_t pi = ((int64_t)s * hkv + g) * np + blockIdx.x;   // partial index

  if (nkeys > 0) {
    // stage K, V rows [t0, t0 + nkeys) and the group's query heads
    const T *kb = kc + (((int64_t)s * hkv + g) * len_max + t0) * D;
    const T *vb = vc + (((int64_t)s * hkv + g) * len_max + t0) * D;
    constexpr int VPR = D / S::kVec;            // 16-byte vectors per row
    constexpr int NIT = kDK * VPR / 256;        // per thread, per tensor
    uint4 kv[NIT], vv[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {          // every load in flight first
      const int x = tid + 256 * it;
      const int r = x / VPR, c = (x % VPR) * S::kVec;
      kv[it] = make_uint4(0, 0, 0, 0);
      vv[it] = make_uint4(0, 0, 0, 0);
      if (r < nkeys) {
        kv[it] = *reinterpret_cast<const uint4 *>(kb + (int64_t)r * D + c);
        vv[it] = *reinterpret_cast<const uint4 *>(vb + (int64_t)r * D + c);
      }
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int x = tid + 256 * it;
      const int r = x / VPR, c = (x % VPR) * S::kVec;
      *reinterpret_cast<uint4 *>(&sm.u.kv.K[r * S::kStr + c]) = kv[it];
      *reinterpret_cast<uint4 *>(&sm.u.kv.V[r * S::kStr + c]) = vv[it];
    }
    for (int x = tid; x < G * D; x += 256)
      sm.Q[x / D][x % D] =
          ldx(q, ((int64_t)s * hq + (int64_t)g * G + x / D) * D + x % D);
    __syncthreads();

    // scores: lane = key, two passes over up to 128 keys, all heads of the wave
    float sc[2][HPW];
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      float acc[HPW];
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) acc[hh] = 0.f;
      const T *kr = &sm.u.kv.K[(lane + 64 * ps) * S::kStr];
      for (int c = 0; c < D; c += 8) {
        float kf[8];
        lds8(kr + c, kf);
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          if (hh >= nh) break;
          const float4 qa = *reinterpret_cast<const float4 *>(&sm.Q[h0 + hh][c]);
          const float4 qb = *reinterpret_cast<const float4 *>(&sm.Q[h0 + hh][c + 4]);
          acc[hh] = fmaf(qa.x, kf[0], acc[hh]);
          acc[hh] = fmaf(qa.y, kf[1], acc[hh]);
          acc[hh] = fmaf(qa.z, kf[2], acc[hh]);
          acc[hh] = fmaf(qa.w, kf[3], acc[hh]);
          acc[hh] = fmaf(qb.x, kf[4], acc[hh]);
          acc[hh] = fmaf(qb.y, kf[5], acc[hh]);
          acc[hh] = fmaf(qb.z, kf[6], acc[hh]);
          acc[hh] = fmaf(qb.w, kf[7], acc[hh]);
        }
      }
      const bool vis = lane + 64 * ps < nkeys;
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) sc[ps][hh] = vis ? acc[hh] * scale_log2 : -INFINITY;
    }
    float mx[HPW], l[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      if (hh >= nh) break;
      mx[hh] = wave_max(fmaxf(sc[0][hh], sc[1][hh]));
      const float p0 = fast_exp2(sc[0][hh] - mx[hh]), p1 = fast_exp2(sc[1][hh] - mx[hh]);
      l[hh] = wave_sum(p0 + p1);
      sm.P[lane][h0 + hh] = p0;
      sm.P[lane + 64][h0 + hh] = p1;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // P.V: lane owns CPL consecutive columns
    float ov[HPW][CPL];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
      for (int u = 0; u < CPL; ++u) ov[hh][u] = 0.f;
    for (int t = 0; t < nkeys; ++t) {
      float vv[CPL];
      if constexpr (CPL == 1) {
        vv[0] = ldx(&sm.u.kv.V[t * S::kStr], lane);
      } else {
#pragma unroll
        for (int u = 0; u < CPL; u += 2)
          lds2(&sm.u.kv.V[t * S::kStr + CPL * lane + u], vv[u], vv[u + 1]);
      }
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        if (hh >= nh) break;
        const float pt = sm.P[t][h0 + hh];
#pragma unroll
        for (int u = 0; u < CPL; ++u) ov[hh][u] = fmaf(pt, vv[u], ov[hh][u]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      if (hh >= nh) break;
      const float inv = 1.f / l[hh];
      float *dst = part_o + (pi * G + h0 + hh) * D + CPL * lane;
#pragma unroll
      for (int u = 0; u < CPL; ++u) dst[u] = ov[hh][u] * inv;
      if (lane == 0) part_lse[pi * G + h0 + hh] = mx[hh] + __log2f(l[hh]);
    }
  } else {
    for (int x = tid; x < G * D; x += 256) part_o[pi * G * D + x] = 0.f;
    if (tid < G) part_lse[pi * G + tid] = -INFINITY;
  }

}

// ---------------------------------------------------------------------------
// bf16, d = 128: matrix-core partials.  Wave w owns keys w*32 .. w*32+31 of
// the item's chunk.
// ---------------------------------------------------------------------------
constexpr int kDecKStr = 128 + 8;    // K row stride in LDS (bf16), 272 B
constexpr int kDecVStr = 128 + 16;   // V row stride in LDS (bf16), 288 B

struct DecMfmaSmem {
  union {
    struct {
      uint16_t Ks[kDK * kDecKStr];
      uint16_t Vs[kDK * kDecVStr];
    } kv;
    struct {                          // after the MFMAs: per-wave partials
      float O[4][16][128];
      float M[4][16], L[4][16];
    } w;
  } u;
};

template <int G>
__global__ __launch_bounds__(256) void decode_attn_mfma(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, int64_t len_max,
    const int64_t *__restrict__ seq_len, int hq, int B,
    const int32_t *__restrict__ sel, int topk, int nsub, float scale_log2,
    float *__restrict__ part_o, float *__restrict__ part_lse) {
  constexpr int D = 128;
  __shared__ DecMfmaSmem sm;
  const int s = blockIdx.z, g = blockIdx.y;
  const int kk = blockIdx.x / nsub, sub = blockIdx.x % nsub;
  const int hkv = gridDim.y, np = gridDim.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, j = lane & 31;

  int64_t len = seq_len[s];
  if (len > len_max) len = len_max;
  const int64_t pos = len - 1;
  const int32_t b = sel[(int64_t)s * topk + kk];
  const int64_t t0 = (int64_t)b * B + (int64_t)sub * kDK;
  int64_t nkeys = (b < 0 || len < 1) ? 0 : pos - t0 + 1;
  if (nkeys > kDK) nkeys = kDK;
  if (nkeys > B - sub * kDK) nkeys = B - sub * kDK;
  const int64_t pi = ((int64_t)s * hkv + g) * np + blockIdx.x;
  if (nkeys <= 0) {
    for (int x = tid; x < G * D; x += 256) part_o[pi * G * D + x] = 0.f;
    if (tid < G) part_lse[pi * G + tid] = -INFINITY;
    return;
  }

  // stage K and V rows (all loads in flight first)
  const uint16_t *kb = kc + (((int64_t)s * hkv + g) * len_max + t0) * D;
  const uint16_t *vb = vc + (((int64_t)s * hkv + g) * len_max + t0) * D;
  u32x4 kr[8], vr[8];
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int x = tid + 256 * it, r = x >> 4, c = (x & 15) * 8;
    kr[it] = u32x4{0u, 0u, 0u, 0u};
    vr[it] = u32x4{0u, 0u, 0u, 0u};
    if (r < nkeys) {
      kr[it] = *reinterpret_cast<const u32x4 *>(kb + (int64_t)r * D + c);
      vr[it] = *reinterpret_cast<const u32x4 *>(vb + (int64_t)r * D + c);
    }
  }
  // query fragments: MFMA column j = query head g*G + j (zero for j >= G)
  bf16x8 qf[8];
  {
    const uint16_t *qp = q + ((int64_t)s * hq + (int64_t)g * G + (j < G ? j : 0)) * D;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (j < G) x = *reinterpret_cast<const u32x4 *>(qp + cc * 16 + 8 * h);
      qf[cc] = as_bf16x8(x);
    }
  }
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int x = tid + 256 * it, r = x >> 4, c = (x & 15) * 8;
    *reinterpret_cast<u32x4 *>(&sm.u.kv.Ks[r * kDecKStr + c]) = kr[it];
    *reinterpret_cast<u32x4 *>(&sm.u.kv.Vs[r * kDecVStr + c]) = vr[it];
  }
  __syncthreads();

  f32x16 acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) acc[cb][rr] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int k0 = wave * 32;
  if (k0 < nkeys) {
    f32x16 sacc;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) sacc[rr] = 0.f;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const u32x4 kraw = *reinterpret_cast<const u32x4 *>(
          &sm.u.kv.Ks[(k0 + j) * kDecKStr + cc * 16 + 8 * h]);
      sacc = mfma32(as_bf16x8(kraw), qf[cc], sacc);
    }
    float x[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int key = k0 + 8 * (rr >> 2) + 4 * h + (rr & 3);
      x[rr] = key < nkeys ? sacc[rr] * scale_log2 : -INFINITY;
    }
    float mloc = x[0];
#pragma unroll
    for (int rr = 1; rr < 16; ++rr) mloc = fmaxf(mloc, x[rr]);
    m = max_with_partner(mloc);          // finite: key k0 is always valid
    f32x8 p0, p1;
    float ps = 0.f;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      p0[rr] = fast_exp2(x[rr] - m);
      p1[rr] = fast_exp2(x[rr + 8] - m);
      ps += p0[rr] + p1[rr];
    }
    l = sum_with_partner(ps);
    const bf16x8 pb0 = __builtin_convertvector(p0, bf16x8);
    const bf16x8 pb1 = __builtin_convertvector(p1, bf16x8);
    const int a16 = lane & 15;
    const uint16_t *vbase = &sm.u.kv.Vs[(k0 + 4 * h + (a16 >> 2)) * kDecVStr +
                                        16 * (j >> 4) + 4 * (a16 & 3)];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const uint16_t *vp = vbase + 16 * ks * kDecVStr + cb * 32;
        const u32x2 lo = lds_read_tr(vp);
        const u32x2 hi = lds_read_tr(vp + 8 * kDecVStr);
        const u32x4 vraw = {lo[0], lo[1], hi[0], hi[1]};
        acc[cb] = mfma32(as_bf16x8(vraw), ks == 0 ? pb0 : pb1, acc[cb]);
      }
    }
  }
  __syncthreads();   // K/V no longer read: the area now holds wave partials
  if (j < G) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        *reinterpret_cast<float4 *>(&sm.u.w.O[wave][j][cb * 32 + 8 * rg + 4 * h]) =
            make_float4(acc[cb][4 * rg], acc[cb][4 * rg + 1], acc[cb][4 * rg + 2],
                        acc[cb][4 * rg + 3]);
    if (h == 0) {
      sm.u.w.M[wave][j] = m;
      sm.u.w.L[wave][j] = l;
    }
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += 256) {
    const int hd = x / D, c = x % D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (w * 32 < nkeys) mm = fmaxf(mm, sm.u.w.M[w][hd]);
    float z = 0.f, ov = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (w * 32 >= nkeys) continue;
      const float sc = fast_exp2(sm.u.w.M[w][hd] - mm);
      z = fmaf(sc, sm.u.w.L[w][hd], z);
      ov = fmaf(sc, sm.u.w.O[w][hd][c], ov);
    }
    part_o[(pi * G + hd) * D + c] = ov / z;
    if (c == 0) part_lse[pi * G + hd] = mm + __log2f(z);
  }
}

// ---------------------------------------------------------------------------
// Merge: one workgroup per (query head, sequence), one thread per column.
// Online log-sum-exp over the np partials, branch-free so the loads of
// consecutive partials can be in flight together.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(D) void decode_merge(
    int np, int G, int hkv, const float *__restrict__ part_o,
    const float *__restrict__ part_lse, float *__restrict__ o,
    float *__restrict__ lse) {
  const int hh = blockIdx.x, s = blockIdx.y, c = threadIdx.x;
  const int hq = gridDim.x, g = hh / G, hl = hh % G;
  const int64_t base = ((int64_t)s * hkv + g) * np;
  float m = -3.0e38f, z = 0.f, acc = 0.f;
#pragma unroll 8
  for (int i = 0; i < np; ++i) {
    const float li = part_lse[(base + i) * G + hl];
    const float oi = part_o[((base + i) * G + hl) * D + c];
    const float mn = fmaxf(m, li);
    const float sc = fast_exp2(m - mn), w = fast_exp2(li - mn);
    z = fmaf(z, sc, w);
    acc = fmaf(acc, sc, w * oi);
    m = mn;
  }
  o[((int64_t)s * hq + hh) * D + c] = acc / z;
  if (lse && c == 0) lse[(int64_t)s * hq + hh] = (m + __log2f(z)) * kLn2;
}

template <typename T, int G, int D>
hipError_t launch_dec(const T *q, const T *kc, const T *vc, int32_t n_seq,
                      int64_t len_max, const int64_t *seq_len, int32_t hq,
                      int32_t hkv, int32_t B, const int32_t *sel, int32_t topk,
                      float scale, float *o, float *lse, float *part_o,
                      float *part_lse, hipStream_t st) {
  const int nsub = (B + kDK - 1) / kDK;
  const dim3 grid(topk * nsub, hkv, n_seq);
  if constexpr (sizeof(T) == 2 && D == 128) {
    hipLaunchKernelGGL((decode_attn_mfma<G>), grid, dim3(256), 0, st, q, kc, vc,
                       len_max, seq_len, hq, B, sel, topk, nsub, scale * kLog2e,
                       part_o, part_lse);
  } else {
    hipLaunchKernelGGL((decode_attn<T, G, D>), grid, dim3(256), 0, st, q, kc, vc,
                       len_max, seq_len, hq, B, sel, topk, nsub, scale * kLog2e,
                       part_o, part_lse);
  }
  hipLaunchKernelGGL((decode_merge<D>), dim3(hq, n_seq), dim3(D), 0, st,
                     topk * nsub, G, hkv, part_o, part_lse, o, lse);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t dec_g(int G, const T *q, const T *kc, const T *vc, int32_t n_seq,
                 int64_t len_max, const int64_t *seq_len, int32_t hq,
                 int32_t hkv, int32_t B, const int32_t *sel, int32_t topk,
                 float scale, float *o, float *lse, float *part_o,
                 float *part_lse, hipStream_t st) {
#define MSA_DEC_CASE(GG)                                                   \
  case GG:                                                                 \
    return launch_dec<T, GG, D>(q, kc, vc, n_seq, len_max, seq_len, hq, hkv, \
                                B, sel, topk, scale, o, lse, part_o,        \
                                part_lse, st);
  switch (G) {
    MSA_DEC_CASE(1)
    MSA_DEC_CASE(2)
    MSA_DEC_CASE(4)
    MSA_DEC_CASE(8)
    MSA_DEC_CASE(16)
    default:
      break;
  }
#undef MSA_DEC_CASE
  return hipErrorInvalidValue;
}

int64_t dec_partials(int32_t n_seq, int32_t hq, int32_t block, int32_t topk) {
  return (int64_t)n_seq * hq * topk * ((block + kDK - 1) / kDK);
}

}  // namespace

bool decode_partials_ok(int32_t dtype, int32_t d, int32_t group, int32_t block,
                        int32_t topk) {
  (void)dtype; (void)d; (void)group; (void)block; (void)topk;
  return true;
}

namespace {

}  // namespace

// Layout: [partial o][partial lse].
size_t decode_ws_bytes(int32_t n_seq, int32_t hq, int32_t d, int32_t block,
                       int32_t topk) {
  const int64_t np = dec_partials(n_seq, hq, block, topk);
  return align256((size_t)np * d * 4) + align256((size_t)np * 4);
}

bool decode_supported(int32_t dtype, int32_t d, int32_t group) {
  const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8 ||
                    group == 16;
  if (!g_ok) return false;
  if (d == 64 || d == 128) return true;
  return d == 256 && dtype == 1;   // fp32 rows of 256 do not fit the LDS stage
}

hipError_t launch_decode(const void *q, const void *k_cache,
                         const void *v_cache, int32_t dtype, int32_t n_seq,
                         int64_t len_max, const int64_t *seq_len, int32_t hq,
                         int32_t hkv, int32_t d, int32_t block,
                         const int32_t *sel, int32_t topk, float scale,
                         float *o, float *lse, void *ws, hipStream_t st) {
  const int G = hq / hkv;
  const int64_t np = dec_partials(n_seq, hq, block, topk);
  char *w = static_cast<char *>(ws);
  float *part_o = reinterpret_cast<float *>(w);
  w += align256((size_t)np * d * 4);
  float *part_lse = reinterpret_cast<float *>(w);
#define MSA_DARGS                                                          \
  n_seq, len_max, seq_len, hq, hkv, block, sel, topk, scale, o, lse, part_o, \
      part_lse, st
  if (dtype == 0) {
    const float *qq = static_cast<const float *>(q);
    const float *kk = static_cast<const float *>(k_cache);
    const float *vv = static_cast<const float *>(v_cache);
    if (d == 64) return dec_g<float, 64>(G, qq, kk, vv, MSA_DARGS);
    if (d == 128) return dec_g<float, 128>(G, qq, kk, vv, MSA_DARGS);
  } else {
    const uint16_t *qq = static_cast<const uint16_t *>(q);
    const uint16_t *kk = static_cast<const uint16_t *>(k_cache);
    const uint16_t *vv = static_cast<const uint16_t *>(v_cache);
    if (d == 64) return dec_g<uint16_t, 64>(G, qq, kk, vv, MSA_DARGS);
    if (d == 128) return dec_g<uint16_t, 128>(G, qq, kk, vv, MSA_DARGS);
    if (d == 256) return dec_g<uint16_t, 256>(G, qq, kk, vv, MSA_DARGS);
  }
#undef MSA_DARGS
  return hipErrorInvalidValue;
}

}  // namespace msa
