// prefill.hip -- sparse-branch prefill: GQA over each query's selected
// blocks, organised KV outer / gather Q (sparse branch of "MiniMax M3模型算力
// 成本大幅降低原因深度解析"; section 2.2 "KV Outer Gather Q：MSA 的关键设计" of
// chenxutan.com's "MiniMax M3 深度实战").
//
// Work is split by the causal structure of the selection.  Row b of the CSR
// holds first the block's own tokens, then (ascending) the later queries that
// chose b.  Two passes:
//   pass A  (block b, KV head g, tile of row b's non-own queries): K[g,b] and
//           V[g,b] are streamed once into LDS per tile and applied to the
//           gathered queries (all G query heads of group g); every (query,
//           head) gets a normalised partial output and its log-sum-exp in the
//           workspace, at the pair's non-own index.
//   pass B  (block b, KV head g, tile of b's own tokens): causal attention
//           inside the own block, then a log-sum-exp merge with the query's
//           partials from pass A, which writes O and LSE.
// The non-own index of CSR position e in row b is e minus the number of own
// entries in rows 0..b, a closed form of the query range.
//
// This file holds the generic VALU kernels (fp32 and bf16 inputs, fp32
// arithmetic); bf16 with d = 128 runs on the MFMA kernel (prefill_mfma.hip).
#include "msa_internal.h"
#include "prefill_common.h"

namespace msa {

int64_t nonown_pairs(int64_t q_pos0, int64_t n_q, int32_t block, int32_t topk) {
  // A token of block b keeps min(K, b + 1) - 1 non-own blocks: b of them for
  // the first K - 1 blocks, K - 1 from block K - 1 on.  Sum the first blocks
  // one by one (at most K - 1 of them), the rest in closed form.
  if (n_q <= 0) return 0;
  const int64_t p0 = q_pos0, p1 = q_pos0 + n_q;       // tokens [p0, p1)
  const int64_t full_from = (int64_t)(topk - 1) * block;   // first token of block K-1
  int64_t total = 0;
  for (int64_t b = p0 / block; b < topk - 1 && b * block < p1; ++b) {
    const int64_t lo = b * block > p0 ? b * block : p0;
    const int64_t hi = (b + 1) * block < p1 ? (b + 1) * block : p1;
    total += (hi - lo) * b;
  }
  const int64_t lo = p0 > full_from ? p0 : full_from;
  if (p1 > lo) total += (p1 - lo) * (int64_t)(topk - 1);
  return total;
}

namespace {

constexpr int kQTA = 4;   // tokens per workgroup (one per wave), generic path
constexpr int kKC = 64;   // keys per chunk

template <typename T>
__device__ __forceinline__ float ld(const T *p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float *p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t *p, int64_t i) {
  return bf16_to_f32(p[i]);
}

template <int G, int D>
struct GenericSmem {
  float Ks[kKC][D + 1];
  float Vs[kKC][D];
  float Qs[kQTA][G][D];
  float Ps[kQTA][G][kKC];
};

// One chunk of (up to) 64 keys for this wave's token: scores, online
// softmax update, and P.V accumulation.  `last` = highest visible key offset
// inside the chunk for this token (keys beyond it are masked).
template <int G, int DU>
__device__ __forceinline__ void chunk_step(GenericSmem<G, 64 * DU> &sm,
                                           int wave, int lane, int last,
                                           float scale_log2, float (&m)[G],
                                           float (&l)[G],
                                           float (&acc)[G][DU]) {
  constexpr int D = 64 * DU;
  float s[G];
#pragma unroll
  for (int h = 0; h < G; ++h) s[h] = 0.f;
  for (int c = 0; c < D; ++c) {
    const float kk = sm.Ks[lane][c];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = fmaf(sm.Qs[wave][h][c], kk, s[h]);
  }
  const bool vis = lane <= last;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float x = vis ? s[h] * scale_log2 : -INFINITY;
    const float mn = fmaxf(m[h], wave_max(x));
    const float alpha = fast_exp2(m[h] - mn);
    const float p = fast_exp2(x - mn);
    l[h] = l[h] * alpha + wave_sum(p);
#pragma unroll
    for (int u = 0; u < DU; ++u) acc[h][u] *= alpha;
    m[h] = mn;
    sm.Ps[wave][h][lane] = p;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int j = 0; j <= last && j < kKC; ++j) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pj = sm.Ps[wave][h][j];
#pragma unroll
      for (int u = 0; u < DU; ++u)
        acc[h][u] = fmaf(pj, sm.Vs[j][lane + 64 * u], acc[h][u]);
    }
  }
}

template <typename T, int G, int DU>
__device__ __forceinline__ void stage_kv(GenericSmem<G, 64 * DU> &sm,
                                         const T *k, const T *v, int64_t row0,
                                         int nrows) {
  constexpr int D = 64 * DU;
  for (int x = threadIdx.x; x < kKC * D; x += 256) {
    const int r = x / D, c = x % D;
    const bool ok = r < nrows;
    sm.Ks[r][c] = ok ? ld(k, (row0 + r) * D + c) : 0.f;
    sm.Vs[r][c] = ok ? ld(v, (row0 + r) * D + c) : 0.f;
  }
}

// Pass A: non-own pairs.  grid = (tile upper bound, Hkv).
template <typename T, int G, int DU>
__global__ __launch_bounds__(256) void prefill_nonown_generic(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    int64_t kv_stride, int64_t q_pos0, int64_t n_q, int hq, int B,
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ q_list,
    const int32_t *__restrict__ tile_ptr, int64_t nb, float scale_log2,
    float *__restrict__ part_o, float *__restrict__ part_lse, int64_t n_part) {
  constexpr int D = 64 * DU;
  __shared__ GenericSmem<G, D> sm;
  const int g = blockIdx.y;
  const int64_t w = blockIdx.x;
  if (w >= tile_ptr[nb]) return;
  const int64_t b = find_row(tile_ptr, nb, w);
  const int64_t t = w - tile_ptr[b];
  const int64_t own_b =
      own_through(b, q_pos0, n_q, B) - own_through(b - 1, q_pos0, n_q, B);
  const int64_t e0 = row_ptr[b] + own_b + t * kQTA;
  const int64_t e_end = row_ptr[b + 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t e = e0 + wave;
  int64_t qi = e < e_end ? q_list[e] : -1;
  const bool active = qi >= 0 && qi < n_q;
  if (!active) qi = 0;
  for (int x = lane; x < G * D; x += 64) {
    const int h = x / D, c = x % D;
    sm.Qs[wave][h][c] = active ? ld(q, (qi * hq + g * G + h) * D + c) : 0.f;
  }
  float m[G], l[G], acc[G][DU];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int u = 0; u < DU; ++u) acc[h][u] = 0.f;
  }
  const T *kb = k + (g * kv_stride) * D;
  const T *vb = v + (g * kv_stride) * D;
  for (int kc = 0; kc < B; kc += kKC) {
    __syncthreads();
    // rows past the key range (only reachable with an invalid selection)
    // are staged as zeros, never read
    int nrows = B - kc < kKC ? B - kc : kKC;             // stay inside block b
    const int64_t room = kv_stride - (b * B + kc);
    if (room < nrows) nrows = room > 0 ? (int)room : 0;
    stage_kv<T, G, DU>(sm, kb, vb, b * B + kc, nrows);
    __syncthreads();
    if (nrows > 0)
      chunk_step<G, DU>(sm, wave, lane, nrows - 1, scale_log2, m, l, acc);
  }
  if (!active) return;
  const int64_t n_idx = e - own_through(b, q_pos0, n_q, B);
  if (n_idx < 0 || n_idx >= n_part) return;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float inv = 1.f / l[h];
    float *dst = part_o + ((n_idx * hq) + g * G + h) * (int64_t)D;
#pragma unroll
    for (int u = 0; u < DU; ++u) dst[lane + 64 * u] = acc[h][u] * inv;
    if (lane == 0) part_lse[n_idx * hq + g * G + h] = m[h] + __log2f(l[h]);
  }
}

// Pass B: own block + merge.  grid = (own tiles, Hkv); own tile w covers
// block b_first + w / (B/4), tokens 4*(w % (B/4)) .. +3 of that block.
template <typename T, int G, int DU>
__global__ __launch_bounds__(256) void prefill_own_generic(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    int64_t kv_stride, int64_t q_pos0, int64_t n_q, int hq, int B,
    const int32_t *__restrict__ sel, int topk,
    const int32_t *__restrict__ slot, float scale_log2,
    const float *__restrict__ part_o, const float *__restrict__ part_lse,
    int64_t n_part, float *__restrict__ o, float *__restrict__ lse) {
  constexpr int D = 64 * DU;
  __shared__ GenericSmem<G, D> sm;
  const int g = blockIdx.y;
  const int tiles_per_block = B / kQTA;
  const int64_t b = q_pos0 / B + blockIdx.x / tiles_per_block;
  const int tt = blockIdx.x % tiles_per_block;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t p = b * B + tt * kQTA + wave;
  const bool active = p >= q_pos0 && p < q_pos0 + n_q;
  int64_t p_hi = b * B + tt * kQTA + kQTA - 1;
  if (p_hi > q_pos0 + n_q - 1) p_hi = q_pos0 + n_q - 1;
  if (p_hi < b * B || b * B + tt * kQTA > q_pos0 + n_q - 1) return;
  const int64_t i = p - q_pos0;
  for (int x = lane; x < G * D; x += 64) {
    const int h = x / D, c = x % D;
    sm.Qs[wave][h][c] = active ? ld(q, (i * hq + g * G + h) * D + c) : 0.f;
  }
  float m[G], l[G], acc[G][DU];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int u = 0; u < DU; ++u) acc[h][u] = 0.f;
  }
  const T *kb = k + (g * kv_stride) * D;
  const T *vb = v + (g * kv_stride) * D;
  const int64_t my_last = (active ? p : b * B) - b * B;   // visible key offset
  const int64_t n_keys = p_hi - b * B + 1;
  for (int64_t kc = 0; kc < n_keys; kc += kKC) {
    __syncthreads();
    const int nrows = (int)(n_keys - kc < kKC ? n_keys - kc : kKC);
    stage_kv<T, G, DU>(sm, kb, vb, b * B + kc, nrows);
    __syncthreads();
    int last = (int)(my_last - kc);
    if (last >= kKC) last = kKC - 1;
    if (last >= 0) chunk_step<G, DU>(sm, wave, lane, last, scale_log2, m, l, acc);
  }
  if (!active) return;
  const int32_t *srow = sel + i * topk;
  const int32_t *xrow = slot + i * topk;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int hh = g * G + h;
    const float own2 = m[h] + __log2f(l[h]);
    float mx = own2;
    for (int kk = 0; kk < topk; ++kk) {
      const int32_t bk = srow[kk];
      if (bk < 0 || bk >= b) continue;
      const int64_t n_idx = xrow[kk] - own_through(bk, q_pos0, n_q, B);
      if (n_idx < 0 || n_idx >= n_part) continue;
      mx = fmaxf(mx, part_lse[n_idx * hq + hh]);
    }
    float z = fast_exp2(own2 - mx);
    float out[DU];
    const float wo = z / l[h];
#pragma unroll
    for (int u = 0; u < DU; ++u) out[u] = acc[h][u] * wo;
    for (int kk = 0; kk < topk; ++kk) {
      const int32_t bk = srow[kk];
      if (bk < 0 || bk >= b) continue;
      const int64_t n_idx = xrow[kk] - own_through(bk, q_pos0, n_q, B);
      if (n_idx < 0 || n_idx >= n_part) continue;
      const float wk = fast_exp2(part_lse[n_idx * hq + hh] - mx);
      z += wk;
      const float *src = part_o + (n_idx * hq + hh) * (int64_t)D;
#pragma unroll
      for (int u = 0; u < DU; ++u) out[u] = fmaf(wk, src[lane + 64 * u], out[u]);
    }
    const float invz = 1.f / z;
    float *dst = o + (i * hq + hh) * (int64_t)D;
#pragma unroll
    for (int u = 0; u < DU; ++u) dst[lane + 64 * u] = out[u] * invz;
    if (lse && lane == 0) lse[i * hq + hh] = (mx + __log2f(z)) * kLn2;
  }
}

template <typename T, int G, int DU>
hipError_t launch_generic(const T *q, const T *k, const T *v, int64_t kv_stride,
                          int64_t q_pos0, int64_t n_q, int hq, int B,
                          const int32_t *sel, int topk, const int32_t *row_ptr,
                          const int32_t *q_list, const int32_t *slot,
                          float scale, float *o, float *lse, int32_t *tile_ptr,
                          float *part_o, float *part_lse, int64_t n_part,
                          hipStream_t st) {
  const int hkv = hq / G;
  const int64_t nb = (q_pos0 + n_q + B - 1) / B;
  const float sl2 = scale * kLog2e;
  if (n_part > 0) {
    const int64_t grid = n_part / kQTA + nb;
    hipLaunchKernelGGL(prefill_tiles, dim3(1), dim3(1024), 0, st, row_ptr,
                       seqtab_one(q_pos0, n_q, B), kQTA, grid, tile_ptr);
    hipLaunchKernelGGL((prefill_nonown_generic<T, G, DU>),
                       dim3((unsigned)grid, hkv), dim3(256), 0, st, q, k, v,
                       kv_stride, q_pos0, n_q, hq, B, row_ptr, q_list, tile_ptr,
                       nb, sl2, part_o, part_lse, n_part);
  }
  const int64_t b_first = q_pos0 / B, b_last = (q_pos0 + n_q - 1) / B;
  const int64_t own_tiles = (b_last - b_first + 1) * (B / kQTA);
  hipLaunchKernelGGL((prefill_own_generic<T, G, DU>),
                     dim3((unsigned)own_tiles, hkv), dim3(256), 0, st, q, k, v,
                     kv_stride, q_pos0, n_q, hq, B, sel, topk, slot, sl2,
                     part_o, part_lse, n_part, o, lse);
  return hipGetLastError();
}

template <typename T, int DU>
hipError_t dispatch_g(int G, const T *q, const T *k, const T *v,
                      int64_t kv_stride, int64_t q_pos0, int64_t n_q, int hq,
                      int B, const int32_t *sel, int topk,
                      const int32_t *row_ptr, const int32_t *q_list,
                      const int32_t *slot, float scale, float *o, float *lse,
                      int32_t *tile_ptr, float *part_o, float *part_lse,
                      int64_t n_part, hipStream_t st) {
#define MSA_G_CASE(GG)                                                       \
  case GG:                                                                   \
    return launch_generic<T, GG, DU>(q, k, v, kv_stride, q_pos0, n_q, hq, B, \
                                     sel, topk, row_ptr, q_list, slot, scale, \
                                     o, lse, tile_ptr, part_o, part_lse,      \
                                     n_part, st);
  switch (G) {
    MSA_G_CASE(1)
    MSA_G_CASE(2)
    MSA_G_CASE(4)
    default:
      break;
  }
  if constexpr (DU <= 2) {
    switch (G) {
      MSA_G_CASE(8)
      MSA_G_CASE(16)
      default:
        break;
    }
  }
#undef MSA_G_CASE
  return hipErrorInvalidValue;
}

}  // namespace

size_t prefill_ws_bytes(int32_t dtype, int64_t q_pos0, int64_t n_q, int32_t hq,
                        int32_t d, int32_t block, int32_t topk) {
  const int64_t nb = (q_pos0 + n_q + block - 1) / block;
  const int64_t np = nonown_pairs(q_pos0, n_q, block, topk);
  if (dtype == 1 && d == 128)   // matrix-core path
    return prefill_chain_ws_bytes(seqtab_one(q_pos0, n_q, block), hq, d, topk);
  // + per-tile metadata of the MFMA pass A, bounded for any head group:
  //   tiles <= pairs / 16 + nb (16 = smallest tile), rows <= pairs + 256 nb.
  return align256((size_t)(nb + 1) * 4) + align256((size_t)np * hq * d * 4) +
         align256((size_t)np * hq * 4) + align256((size_t)(np / 16 + nb) * 16) +
         align256((size_t)(np + 256 * nb) * 4);
}

bool generic_prefill_supported(int32_t d, int32_t group) {
  const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8 ||
                    group == 16;
  if (!g_ok) return false;
  if (d == 64 || d == 128) return true;
  if (d == 256) return group <= 4;   // LDS: K, V, Q and P tiles in fp32
  return false;
}

hipError_t launch_prefill_generic(const void *q, const void *k, const void *v,
                                  int32_t dtype, int64_t kv_stride,
                                  int64_t q_pos0, int64_t n_q, int32_t hq,
                                  int32_t hkv, int32_t d, int32_t block,
                                  const int32_t *sel, int32_t topk,
                                  const int32_t *row_ptr,
                                  const int32_t *q_list, const int32_t *slot,
                                  float scale, float *o, float *lse, void *ws,
                                  hipStream_t st) {
  const int G = hq / hkv;
  const int64_t nb = (q_pos0 + n_q + block - 1) / block;
  const int64_t np = nonown_pairs(q_pos0, n_q, block, topk);
  char *w = static_cast<char *>(ws);
  int32_t *tile_ptr = reinterpret_cast<int32_t *>(w);
  w += align256((size_t)(nb + 1) * 4);
  float *part_o = reinterpret_cast<float *>(w);
  w += align256((size_t)np * hq * d * 4);
  float *part_lse = reinterpret_cast<float *>(w);
#define MSA_ARGS                                                              \
  kv_stride, q_pos0, n_q, hq, block, sel, topk, row_ptr, q_list, slot, scale, \
      o, lse, tile_ptr, part_o, part_lse, np, st
  if (dtype == 0) {
    const float *qq = static_cast<const float *>(q);
    const float *kk = static_cast<const float *>(k);
    const float *vv = static_cast<const float *>(v);
    if (d == 64) return dispatch_g<float, 1>(G, qq, kk, vv, MSA_ARGS);
    if (d == 128) return dispatch_g<float, 2>(G, qq, kk, vv, MSA_ARGS);
    if (d == 256) return dispatch_g<float, 4>(G, qq, kk, vv, MSA_ARGS);
  } else {
    const uint16_t *qq = static_cast<const uint16_t *>(q);
    const uint16_t *kk = static_cast<const uint16_t *>(k);
    const uint16_t *vv = static_cast<const uint16_t *>(v);
    if (d == 64) return dispatch_g<uint16_t, 1>(G, qq, kk, vv, MSA_ARGS);
    if (d == 128) return dispatch_g<uint16_t, 2>(G, qq, kk, vv, MSA_ARGS);
    if (d == 256) return dispatch_g<uint16_t, 4>(G, qq, kk, vv, MSA_ARGS);
  }
#undef MSA_ARGS
  return hipErrorInvalidValue;
}

}  // namespace msa
