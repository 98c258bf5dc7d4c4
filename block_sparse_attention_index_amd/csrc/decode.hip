// decode.hip -- sparse-branch decode: one new query per sequence attends to
// its selected blocks (decode part of section 3.3 of chenxutan.com's "MiniMax
// M3 深度实战"; GQA over the chosen blocks only, sparse branch of "MiniMax M3
// 模型算力成本大幅降低原因深度解析").
//
// Split-KV: work item = (sequence, KV head, selected block, chunk of 64 keys),
// so even one sequence fills the chip.  Each item streams its K/V rows once
// (for all G query heads of the group), writes a normalised partial output
// and its base-2 log-sum-exp; a second kernel merges the partials of each
// (sequence, head) by log-sum-exp.  HBM-bound: K and V are read once.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kDK = 64;   // keys per work item

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

template <int G, int D>
struct DecSmem {
  float Ks[kDK][D + 1];
  float Vs[kDK][D];
  float Qs[G][D];
  float Ps[4][kDK];
};

// grid = (topk * nsub, Hkv, n_seq)
template <typename T, int G, int DU>
__global__ __launch_bounds__(256) void decode_partial_generic(
    const T *__restrict__ q, const T *__restrict__ kc, const T *__restrict__ vc,
    int64_t len_max, const int64_t *__restrict__ seq_len, int hq, int B,
    const int32_t *__restrict__ sel, int topk, int nsub, float scale_log2,
    float *__restrict__ part_o, float *__restrict__ part_lse) {
  constexpr int D = 64 * DU;
  __shared__ DecSmem<G, D> sm;
  const int s = blockIdx.z, g = blockIdx.y;
  const int kk = blockIdx.x / nsub, sub = blockIdx.x % nsub;
  const int hkv = gridDim.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int64_t len = seq_len[s];
  if (len > len_max) len = len_max;
  const int64_t pos = len - 1;
  const int32_t b = sel[(int64_t)s * topk + kk];
  const int64_t t0 = (int64_t)b * B + (int64_t)sub * kDK;
  int64_t nkeys = b < 0 ? 0 : pos - t0 + 1;
  if (nkeys > kDK) nkeys = kDK;
  if (nkeys > B - sub * kDK) nkeys = B - sub * kDK;   // stay inside block b
  const int64_t pi = (((int64_t)s * hkv + g) * topk + kk) * nsub + sub;
  if (nkeys <= 0 || b * (int64_t)B > pos) {
    for (int x = threadIdx.x; x < G * D; x += 256)
      part_o[pi * G * D + x] = 0.f;
    if (threadIdx.x < G) part_lse[pi * G + threadIdx.x] = -INFINITY;
    return;
  }
  const T *kb = kc + ((int64_t)s * hkv + g) * len_max * D;
  const T *vb = vc + ((int64_t)s * hkv + g) * len_max * D;
  for (int x = threadIdx.x; x < kDK * D; x += 256) {
    const int r = x / D, c = x % D;
    const bool ok = r < nkeys;
    sm.Ks[r][c] = ok ? ldx(kb, (t0 + r) * D + c) : 0.f;
    sm.Vs[r][c] = ok ? ldx(vb, (t0 + r) * D + c) : 0.f;
  }
  for (int x = threadIdx.x; x < G * D; x += 256)
    sm.Qs[x / D][x % D] =
        ldx(q, ((int64_t)s * hq + (int64_t)g * G + x / D) * D + x % D);
  __syncthreads();
  for (int h = wave; h < G; h += 4) {
    float acc = 0.f;
    for (int c = 0; c < D; ++c) acc = fmaf(sm.Qs[h][c], sm.Ks[lane][c], acc);
    const float x = lane < nkeys ? acc * scale_log2 : -INFINITY;
    const float mx = wave_max(x);
    const float p = fast_exp2(x - mx);
    const float l = wave_sum(p);
    sm.Ps[wave][lane] = p;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float o[DU];
#pragma unroll
    for (int u = 0; u < DU; ++u) o[u] = 0.f;
    for (int j = 0; j < nkeys; ++j) {
      const float pj = sm.Ps[wave][j];
#pragma unroll
      for (int u = 0; u < DU; ++u) o[u] = fmaf(pj, sm.Vs[j][lane + 64 * u], o[u]);
    }
    const float inv = 1.f / l;
    float *dst = part_o + (pi * G + h) * D;
#pragma unroll
    for (int u = 0; u < DU; ++u) dst[lane + 64 * u] = o[u] * inv;
    if (lane == 0) part_lse[pi * G + h] = mx + __log2f(l);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// grid = (Hkv, n_seq); wave w merges heads w, w+4, ... of the group.
template <int G, int DU>
__global__ __launch_bounds__(256) void decode_merge_generic(
    int hq, int np, const float *__restrict__ part_o,
    const float *__restrict__ part_lse, float *__restrict__ o,
    float *__restrict__ lse) {
  constexpr int D = 64 * DU;
  const int g = blockIdx.x, s = blockIdx.y, hkv = gridDim.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t base = ((int64_t)s * hkv + g) * np;   // first partial
  for (int h = wave; h < G; h += 4) {
    float mx = -INFINITY;
    for (int j = 0; j < np; ++j) mx = fmaxf(mx, part_lse[(base + j) * G + h]);
    float z = 0.f, acc[DU];
#pragma unroll
    for (int u = 0; u < DU; ++u) acc[u] = 0.f;
    for (int j = 0; j < np; ++j) {
      const float lj = part_lse[(base + j) * G + h];
      if (lj == -INFINITY) continue;
      const float w = fast_exp2(lj - mx);
      z += w;
      const float *src = part_o + ((base + j) * G + h) * D;
#pragma unroll
      for (int u = 0; u < DU; ++u) acc[u] = fmaf(w, src[lane + 64 * u], acc[u]);
    }
    const float inv = 1.f / z;
    const int64_t hh = (int64_t)s * hq + (int64_t)g * G + h;
#pragma unroll
    for (int u = 0; u < DU; ++u) o[hh * D + lane + 64 * u] = acc[u] * inv;
    if (lse && lane == 0) lse[hh] = (mx + __log2f(z)) * kLn2;
  }
}

template <typename T, int G, int DU>
hipError_t launch_dec(const T *q, const T *kc, const T *vc, int32_t n_seq,
                      int64_t len_max, const int64_t *seq_len, int32_t hq,
                      int32_t hkv, int32_t B, const int32_t *sel, int32_t topk,
                      float scale, float *o, float *lse, float *part_o,
                      float *part_lse, hipStream_t st) {
  const int nsub = (B + kDK - 1) / kDK;
  hipLaunchKernelGGL((decode_partial_generic<T, G, DU>),
                     dim3(topk * nsub, hkv, n_seq), dim3(256), 0, st, q, kc, vc,
                     len_max, seq_len, hq, B, sel, topk, nsub, scale * kLog2e,
                     part_o, part_lse);
  hipLaunchKernelGGL((decode_merge_generic<G, DU>), dim3(hkv, n_seq), dim3(256),
                     0, st, hq, topk * nsub, part_o, part_lse, o, lse);
  return hipGetLastError();
}

template <typename T, int DU>
hipError_t dec_g(int G, const T *q, const T *kc, const T *vc, int32_t n_seq,
                 int64_t len_max, const int64_t *seq_len, int32_t hq,
                 int32_t hkv, int32_t B, const int32_t *sel, int32_t topk,
                 float scale, float *o, float *lse, float *part_o,
                 float *part_lse, hipStream_t st) {
#define MSA_DEC_CASE(GG)                                                     \
  case GG:                                                                   \
    return launch_dec<T, GG, DU>(q, kc, vc, n_seq, len_max, seq_len, hq, hkv, \
                                 B, sel, topk, scale, o, lse, part_o,         \
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

}  // namespace

size_t decode_ws_bytes(int32_t n_seq, int32_t hq, int32_t d, int32_t block,
                       int32_t topk) {
  const int64_t np = (int64_t)n_seq * hq * topk * ((block + kDK - 1) / kDK);
  return align256((size_t)np * d * 4) + align256((size_t)np * 4);
}

bool decode_supported(int32_t dtype, int32_t d, int32_t group) {
  (void)dtype;
  const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8 ||
                    group == 16;
  return g_ok && (d == 64 || d == 128 || d == 256);
}

hipError_t launch_decode(const void *q, const void *k_cache,
                         const void *v_cache, int32_t dtype, int32_t n_seq,
                         int64_t len_max, const int64_t *seq_len, int32_t hq,
                         int32_t hkv, int32_t d, int32_t block,
                         const int32_t *sel, int32_t topk, float scale,
                         float *o, float *lse, void *ws, hipStream_t st) {
  const int G = hq / hkv;
  const int64_t np = (int64_t)n_seq * hq * topk * ((block + kDK - 1) / kDK);
  float *part_o = static_cast<float *>(ws);
  float *part_lse = reinterpret_cast<float *>(static_cast<char *>(ws) +
                                              align256((size_t)np * d * 4));
#define MSA_DARGS                                                          \
  n_seq, len_max, seq_len, hq, hkv, block, sel, topk, scale, o, lse, part_o, \
      part_lse, st
  if (dtype == 0) {
    const float *qq = static_cast<const float *>(q);
    const float *kk = static_cast<const float *>(k_cache);
    const float *vv = static_cast<const float *>(v_cache);
    if (d == 64) return dec_g<float, 1>(G, qq, kk, vv, MSA_DARGS);
    if (d == 128) return dec_g<float, 2>(G, qq, kk, vv, MSA_DARGS);
    if (d == 256) return dec_g<float, 4>(G, qq, kk, vv, MSA_DARGS);
  } else {
    const uint16_t *qq = static_cast<const uint16_t *>(q);
    const uint16_t *kk = static_cast<const uint16_t *>(k_cache);
    const uint16_t *vv = static_cast<const uint16_t *>(v_cache);
    if (d == 64) return dec_g<uint16_t, 1>(G, qq, kk, vv, MSA_DARGS);
    if (d == 128) return dec_g<uint16_t, 2>(G, qq, kk, vv, MSA_DARGS);
    if (d == 256) return dec_g<uint16_t, 4>(G, qq, kk, vv, MSA_DARGS);
  }
#undef MSA_DARGS
  return hipErrorInvalidValue;
}

}  // namespace msa
