// decode.hip -- sparse-branch decode: one new query per sequence attends to
// its selected blocks (decode part of section 3.3 of chenxutan.com's "MiniMax
// M3 深度实战"; GQA over the chosen blocks only, sparse branch of "MiniMax M3
// 模型算力成本大幅降低原因深度解析").
//
// Split-KV: the selected blocks of every (sequence, KV head) are cut into
// units whose normalised partial outputs and base-2 log-sum-exps are merged
// per (sequence, query head).  The attention calls merge in a second kernel;
// the fused decode step merges inside the streaming kernel, the last
// workgroup of each run combining the run's records, which are written and
// read with device-coherent (SC1) accesses and ordered by an arrival counter
// -- no cache write-back or invalidate (a release fence per workgroup cost
// more than the second launch).  bf16 with d = 128 runs a persistent
// streaming kernel on the matrix cores (one workgroup per CU, K/V chunks
// arriving by LDS DMA while the previous chunk computes); other shapes use a
// VALU kernel with one work item per (sequence, KV head, selected block,
// 128-key chunk).  HBM-bound: K and V are read once.
#include <mutex>
#include <type_traits>

#include "msa_internal.h"
#include "index_common.h"
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
// bf16, d = 128: persistent streaming kernel on the matrix cores.
//
// Work unit u = ((s * Hkv + g) * topk + kk) * nseg + seg: keys
// [b*B + seg*seg_len, +seg_len) of block b = sel[s][kk], clipped to the block
// and to the query position.  One
// workgroup per CU walks a contiguous range of units as one stream of 128-key
// chunks: each chunk's K and V rows arrive by LDS DMA (16 bytes per lane,
// XOR-swizzled 256-byte rows) into one of two buffers while the previous
// chunk is computed, and the next unit's queries are staged with its first
// chunk.  Wave w owns keys 32w .. 32w+31 of a chunk: S^T = K Q^T with the G
// heads as MFMA columns, an online softmax per head, O^T += V^T P^T with V^T
// read by ds_read_b64_tr_b16.  The softmax state carries on across the
// consecutive units of one (sequence, KV head) -- a run; at a run's last
// chunk the four waves' (max, sum, O) are combined through LDS (reusing the
// chunk buffer just consumed) into the run's normalised partial and base-2
// log-sum-exp, record `first unit of the run in this range` of the workspace
// (decode_merge_runs finds them from the static unit partition).  The
// two buffers are distinct LDS objects named statically by each chunk step,
// so the compiler can tell the DMA into one from the reads of the other.
// ---------------------------------------------------------------------------
constexpr int kSK = 128;   // keys per streamed chunk (one per wave quarter)
constexpr float kDecLazy = 8.f;   // reference-max slack (log2 units)

struct StreamBuf {
  uint16_t Ks[kSK * 128];
  uint16_t Vs[kSK * 128];
};

typedef __attribute__((address_space(1))) void *dec_gptr_t;
typedef __attribute__((address_space(3))) void *dec_lptr_t;

// K: segment sg of row r at slot sg ^ (r & 15) (a 16-lane A-operand read hits
// 16 bank groups); V: at slot sg ^ 2(r & 7) (a transposed-read group's 4 rows
// x 2 segments are distinct slots, and rows 8 apart share the pattern).
__device__ __forceinline__ int dkswz(int r, int sg) { return sg ^ (r & 15); }
__device__ __forceinline__ int dvswz(int r, int sg) { return sg ^ (2 * (r & 7)); }

struct DecUnit {
  int s, g;
  int64_t t0;    // first key of the unit
  int64_t kvo;   // element offset of that key's K (and V) row
  int nk;        // keys in the unit (0: empty)
};

// FUSED: the step of msa_decode_step -- the query sits at position
// seq_len[s] (its key was just appended), and the selection is merged here
// from the scan's per-chunk candidate lists (cand_s, cand_b): every workgroup
// merges the rows of the (at most kStepSeqs) sequences its units belong to,
// and the workgroup holding a sequence's first unit also writes the row to
// `sel`.  Otherwise the query sits at seq_len[s] - 1 and `sel` is read.
constexpr int kStepSeqs = 8;

// Device-coherent accesses to the decode partial records of the fused step.
// A record is written with vector buffer stores carrying the SC1 cache-policy
// bit (device scope: written through to the point where every XCD's L2 sees
// it) and read back by another workgroup, on any XCD, with SC1 buffer loads,
// which do not hit a stale L2 line.  Ordering: the writer waits for its
// stores to complete before its workgroup's arrival is counted; the reader
// loads only after the count says every writer has arrived.  No L2
// write-back or invalidate is needed (both cost far more per workgroup).
constexpr int kSc1 = 16;   // cache-policy operand: SC1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t record_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}
typedef unsigned u32v4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(
      u32v4{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)},
      r, off, 0, kSc1);
}
__device__ __forceinline__ void store_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, kSc1);
}
__device__ __forceinline__ float4 load4_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32v4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1);
  return make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                     __uint_as_float(x.w));
}
__device__ __forceinline__ float load_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kSc1));
}

// Workgroup of the static unit partition (u_q units each, one more for the
// first u_r) that holds unit u.
__device__ __forceinline__ uint32_t unit_wg(uint32_t u, uint32_t u_q, uint32_t u_r) {
  const uint32_t split = u_r * (u_q + 1);   // units of the longer ranges
  return u < split ? u / (u_q + 1) : u_r + (u - split) / u_q;
}

// Combine of run sg's partials inside the streaming kernel, by the last
// workgroup to finish its part of the run: the workgroups b0..b1 whose unit
// ranges meet the run each left one normalised partial and base-2
// log-sum-exp (device-coherent records), in the slot of their first unit in
// the run.  Thread t owns four consecutive columns of one query head; the
// partials' loads go out in batches of kBatch so their round trips overlap.
template <int G>
__device__ __forceinline__ void combine_run(uint32_t sg, uint32_t ups_g, uint32_t u_q,
                                            uint32_t u_r, int hq, int hkv,
                                            const float *__restrict__ part_o,
                                            const float *__restrict__ part_lse,
                                            float *__restrict__ o, float *__restrict__ lse) {
  constexpr int D = 128;
  constexpr int kBatch = 16;
  const uint32_t u0 = sg * ups_g, u1 = u0 + ups_g - 1;
  const uint32_t b0 = unit_wg(u0, u_q, u_r), b1 = unit_wg(u1, u_q, u_r);
  const int s = (int)(sg / (uint32_t)hkv), g = (int)(sg - (uint32_t)s * (uint32_t)hkv);
  for (int x = threadIdx.x; x < G * D / 4; x += 256) {
    const int hd = x / (D / 4), c4 = (x % (D / 4)) * 4;
    float m = -3.0e38f, z = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (uint32_t bx0 = b0; bx0 <= b1; bx0 += kBatch) {
      float li[kBatch];
      float4 oi[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const uint32_t bx = bx0 + k;
        li[k] = -INFINITY;
        oi[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (bx <= b1) {
          const uint32_t ub = bx * u_q + (bx < u_r ? bx : u_r);
          const size_t sl = ub > u0 ? ub : u0;
          li[k] = load_sc1(record_rsrc(part_lse + sl * G, G * 4), hd * 4);
          oi[k] = load4_sc1(record_rsrc(part_o + sl * G * D, G * D * 4), (hd * D + c4) * 4);
        }
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const float mn = fmaxf(m, li[k]);
        const float sc = fast_exp2(m - mn), w = fast_exp2(li[k] - mn);
        z = fmaf(z, sc, w);
        acc.x = fmaf(acc.x, sc, w * oi[k].x);
        acc.y = fmaf(acc.y, sc, w * oi[k].y);
        acc.z = fmaf(acc.z, sc, w * oi[k].z);
        acc.w = fmaf(acc.w, sc, w * oi[k].w);
        m = mn;
      }
    }
    const int64_t hh = (int64_t)s * hq + (int64_t)g * G + hd;
    *reinterpret_cast<float4 *>(&o[hh * D + c4]) =
        make_float4(acc.x / z, acc.y / z, acc.z / z, acc.w / z);
    if (lse && c4 == 0) lse[hh] = (m + __log2f(z)) * kLn2;
  }
}

template <int G, bool FUSED>
__global__ __launch_bounds__(256) void decode_stream(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, int64_t len_max, const int32_t *__restrict__ ptab,
    int pt_stride, int64_t n_pages, const int64_t *__restrict__ seq_len, int hq, int hkv, int B,
    int32_t *__restrict__ sel, int topk, int nseg, int seg_len,
    uint32_t u_q, uint32_t u_r, float scale_log2, float *__restrict__ part_o,
    float *__restrict__ part_lse, const float *__restrict__ cand_s,
    const int *__restrict__ cand_b, int n_chunks, int64_t nb_max,
    int *__restrict__ run_cnt, float *__restrict__ o, float *__restrict__ lse) {
  constexpr int D = 128;
  constexpr int QE = G * D < 512 ? 512 : G * D;   // staged query elements
  __shared__ StreamBuf sb0;
  __shared__ StreamBuf sb1;
  __shared__ uint16_t qs[QE];
  __shared__ int32_t selrows[FUSED ? kStepSeqs * 64 : 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, j = lane & 31;

  // units [u_begin, u_end): u_q each, one more for the first u_r workgroups
  // (32-bit unit arithmetic: the host keeps the unit count below 2^31)
  const uint32_t bx = blockIdx.x;
  const uint32_t u_begin = bx * u_q + (bx < u_r ? bx : u_r);
  const uint32_t u_end = u_begin + u_q + (bx < u_r ? 1u : 0u);
  const uint32_t ups = (uint32_t)(hkv * topk * nseg);   // units per sequence
  const uint32_t s_first = u_begin / ups;
  // the query's length (keys 0 .. len-1 are visible)
  auto query_len = [&](uint32_t s) __attribute__((always_inline)) {
    int64_t len = seq_len[s] + (FUSED ? 1 : 0);
    return len > len_max ? len_max : len;
  };
  // element offset of key b * B + off of sequence s, KV head g: contiguous
  // [n_seq][Hkv][len_max][d] caches, or (ptab) the page of block b in
  // [n_pages][Hkv][B][d] pools; -1 when the block has no page
  auto kv_offset = [&](int s, int g, int64_t b, int64_t off) __attribute__((always_inline)) {
    if (ptab) {
      const int32_t pg = b < pt_stride ? ptab[(int64_t)s * pt_stride + b] : -1;
      if (pg < 0 || pg >= n_pages) return (int64_t)-1;
      return (((int64_t)pg * hkv + g) * B + off) * D;
    }
    return (((int64_t)s * hkv + g) * len_max + b * B + off) * D;
  };

  // Unit u of (sequence, KV head) sg = u / (topk * nseg): segment-major, and
  // within a segment the selection's last entry first -- the own block when
  // the row is full -- then ranks 0 .. topk-2.  So a range that starts on a
  // segment boundary starts on an own-block unit, whose block is known
  // before the selection is.
  auto unit_pos = [&](uint32_t u, int &s, int &g, int &seg, int &kk) __attribute__((always_inline)) {
    const uint32_t upg = (uint32_t)(topk * nseg);
    const uint32_t sg = u / upg, idx = u - sg * upg;
    seg = (int)(idx / (uint32_t)topk);
    const int kr = (int)(idx - (uint32_t)seg * (uint32_t)topk);
    kk = kr == 0 ? topk - 1 : kr - 1;
    s = (int)(sg / (uint32_t)hkv);
    g = (int)(sg - (uint32_t)s * (uint32_t)hkv);
  };
  auto unit = [&](uint32_t u) __attribute__((always_inline)) {
    DecUnit d;
    int seg, kk;
    unit_pos(u, d.s, d.g, seg, kk);
    const int64_t len = query_len(d.s);
    int32_t b;
    if constexpr (FUSED)
      b = ((uint32_t)d.s - s_first < kStepSeqs) ? selrows[((uint32_t)d.s - s_first) * 64 + kk] : -1;
    else
      b = sel[(int64_t)d.s * topk + kk];
    d.t0 = (int64_t)b * B + (int64_t)seg * seg_len;
    int64_t n = (b < 0 || len < 1) ? 0 : len - d.t0;   // keys t0 .. len-1
    if (n > seg_len) n = seg_len;
    if (n > (int64_t)B - (int64_t)seg * seg_len) n = (int64_t)B - (int64_t)seg * seg_len;
    d.kvo = n > 0 ? kv_offset(d.s, d.g, b, (int64_t)seg * seg_len) : -1;
    d.nk = n > 0 && d.kvo >= 0 ? (int)n : 0;
    return d;
  };
  // first non-empty unit at or after u (empty ones get their neutral
  // partial: o = 0, lse = -inf)
  auto next_unit = [&](uint32_t u, DecUnit &d) __attribute__((always_inline)) {
    for (; u < u_end; ++u) {
      d = unit(u);
      if (d.nk > 0) break;
    }
    return u;
  };
  // Runs: the units of one (sequence, KV head) in this workgroup's range
  // share the query rows, so the online softmax simply continues across them
  // and one partial per run is written, in the slot of the run's first unit
  // in the range (unique per workgroup and run, below n_units).  A run whose
  // units are all empty gets the neutral partial (o = 0, lse = -inf).
  const uint32_t ups_g = (uint32_t)(topk * nseg);   // units per (sequence, KV head)
  auto run_slot = [&](uint32_t sg) __attribute__((always_inline)) {
    const uint32_t u0 = sg * ups_g;
    return u0 > u_begin ? u0 : u_begin;
  };
  // FUSED: the run's workgroups meet here once each has stored its partial
  // (device-coherent stores, completed by each wave before the barrier); the
  // last to arrive combines them into o and lse (the counters were zeroed by
  // the scan kernel).
  __shared__ int last_arrival;
  auto arrive = [&](uint32_t sg) __attribute__((always_inline)) {
    if constexpr (FUSED) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) {
        const uint32_t n_wg = unit_wg(sg * ups_g + ups_g - 1, u_q, u_r) -
                              unit_wg(sg * ups_g, u_q, u_r) + 1;
        const int before = __hip_atomic_fetch_add(&run_cnt[sg], 1, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        last_arrival = before == (int)n_wg - 1;
      }
      __syncthreads();
      if (last_arrival) combine_run<G>(sg, ups_g, u_q, u_r, hq, hkv, part_o, part_lse, o, lse);
    }
  };
  auto put_neutral = [&](uint32_t sg) __attribute__((always_inline)) {
    const size_t sl = run_slot(sg);
    if constexpr (FUSED) {
      const __amdgpu_buffer_rsrc_t ro = record_rsrc(part_o + sl * G * D, G * D * 4);
      const __amdgpu_buffer_rsrc_t rl = record_rsrc(part_lse + sl * G, G * 4);
      for (int x4 = tid; x4 < G * D / 4; x4 += 256)
        store_sc1(ro, x4 * 16, make_float4(0.f, 0.f, 0.f, 0.f));
      if (tid < G) store_sc1(rl, tid * 4, -INFINITY);
    } else {
      for (int x = tid; x < G * D; x += 256) part_o[sl * G * D + x] = 0.f;
      if (tid < G) part_lse[sl * G + tid] = -INFINITY;
    }
    arrive(sg);
  };
  uint32_t sg_next = u_begin / ups_g;   // runs before this one are written
  // rows row0 .. row0 + nrows - 1 of the unit (from its first key)
  auto dma_kv = [&](StreamBuf &buf, const DecUnit &d, int64_t row0, int nrows)
      __attribute__((always_inline)) {
    const uint16_t *kb = kc + d.kvo + row0 * D;
    const uint16_t *vb = vc + d.kvo + row0 * D;
    constexpr int IPW = (kSK * D / 8) / 256;   // instructions per wave per tensor
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int inst = wave * IPW + i;
      const int pslot = inst * 64 + lane;          // 16-byte slot in the chunk
      const int r = pslot >> 4, sp = pslot & 15;
      const int64_t rr = r < nrows ? r : nrows - 1;   // rows past the end repeat the last
      __builtin_amdgcn_global_load_lds(
          (dec_gptr_t)(const_cast<uint16_t *>(kb + rr * D + dkswz(r, sp) * 8)),
          (dec_lptr_t)(&buf.Ks[inst * 64 * 8]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          (dec_gptr_t)(const_cast<uint16_t *>(vb + rr * D + dvswz(r, sp) * 8)),
          (dec_lptr_t)(&buf.Vs[inst * 64 * 8]), 16, 0, 0);
    }
  };
  // the unit's G query rows (contiguous in q) copied as they are
  auto dma_q = [&](const DecUnit &d) __attribute__((always_inline)) {
    if (wave == 0) {
      const uint16_t *qb = q + ((int64_t)d.s * hq + (int64_t)d.g * G) * D;
#pragma unroll
      for (int i = 0; i < QE / 512; ++i) {
        const int off = (i * 512 + lane * 8) % (G * D);
        __builtin_amdgcn_global_load_lds((dec_gptr_t)(const_cast<uint16_t *>(qb + off)),
                                         (dec_lptr_t)(&qs[i * 512]), 16, 0, 0);
      }
    }
  };
  auto kv_rows = [&](int n) __attribute__((always_inline)) { return n < kSK ? n : kSK; };

  // FUSED: the first unit's queries and chunk go out before the selection
  // merge when that unit is an own-block one (the own block is the row's
  // last entry once the row is full, own >= topk - 1)
  bool pre = false;
  if constexpr (FUSED) {
    if (u_begin < u_end) {
      DecUnit d0;
      int seg0, kk0;
      unit_pos(u_begin, d0.s, d0.g, seg0, kk0);
      const int64_t len0 = query_len(d0.s);
      const int64_t own0 = len0 >= 1 ? (len0 - 1) / B : 0;
      if (kk0 == topk - 1 && len0 >= 1 && own0 >= topk - 1 && own0 < nb_max) {
        d0.t0 = own0 * B + (int64_t)seg0 * seg_len;
        int64_t n0 = len0 - d0.t0;
        if (n0 > seg_len) n0 = seg_len;
        if (n0 > (int64_t)B - (int64_t)seg0 * seg_len) n0 = (int64_t)B - (int64_t)seg0 * seg_len;
        d0.kvo = n0 > 0 ? kv_offset(d0.s, d0.g, own0, (int64_t)seg0 * seg_len) : -1;
        if (n0 > 0 && d0.kvo >= 0) {
          d0.nk = (int)n0;
          dma_q(d0);
          dma_kv(sb0, d0, 0, kv_rows(d0.nk));
          pre = true;
        }
      }
    }
  }
  if constexpr (FUSED) {
    if (u_begin < u_end) {
      const uint32_t s_last = (u_end - 1) / ups;
      for (uint32_t s = s_first + wave; s <= s_last && s - s_first < kStepSeqs; s += 4) {
        const int64_t len = query_len(s);   // in flight with the lists' loads
        int32_t *row = &selrows[(s - s_first) * 64];
        // scratch: a quarter of the (still unused) second chunk buffer per
        // wave -- the first may already be receiving the first unit's chunk
        float *st_s = reinterpret_cast<float *>(&sb1) + wave * (int)(sizeof(StreamBuf) / 16);
        int *st_b = reinterpret_cast<int *>(st_s) + (int)(sizeof(StreamBuf) / 32);
        const size_t c0 = (size_t)s * n_chunks * (topk - 1);
        decode_merge_lists(
            cand_s + c0, cand_b + c0, n_chunks, topk, 1,
            [&] {
              int64_t own = len >= 1 ? (len - 1) / B : 0;
              return (int)(own >= nb_max ? nb_max - 1 : own);
            },
            row, st_s, st_b, (int)(sizeof(StreamBuf) / 32));
        if (s * ups >= u_begin) {   // this workgroup holds the sequence's first unit
          __builtin_amdgcn_s_waitcnt(0xC07F);   // the row's LDS writes have landed
          if (lane < topk) sel[(size_t)s * topk + lane] = row[lane];
        }
      }
    }
    __syncthreads();
  }

  DecUnit cu;
  uint32_t u = next_unit(u_begin, cu);
  if (u >= u_end) {
    for (uint32_t sg = sg_next; sg <= (u_end - 1) / ups_g; ++sg) put_neutral(sg);
    return;
  }
  DecUnit nu = cu;
  uint32_t un = next_unit(u + 1, nu);
  if (!(pre && u == u_begin)) {   // else the same unit's chunk is already on its way
    dma_q(cu);
    dma_kv(sb0, cu, 0, kv_rows(cu.nk));
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // V^T operand offsets (bytes), per column block: the 16-lane group reads 4
  // keys x 16 columns of this wave's 32 keys; lane a16 supplies key a16/4 and
  // the 8-byte piece a16%4.  (One offset per column block, every read a
  // constant away from it, keeps the compiler's alias information.)
  int voff[4];
  {
    const int a16 = lane & 15;
    const int vrow = wave * 32 + 4 * h + (a16 >> 2);
    const int vcol0 = 16 * (j >> 4) + 4 * (a16 & 3);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int col = cb * 32 + vcol0;
      voff[cb] = (vrow * D + dvswz(vrow, col >> 3) * 8 + (col & 7)) * 2;
    }
  }

  bf16x8 qf[8];
  f32x16 acc[4];
  float m = -INFINITY, l = 0.f;
  int ci = 0;

  auto chunk = [&](auto tag) __attribute__((always_inline)) {
    constexpr int P = decltype(tag)::value;
    StreamBuf &cur = P ? sb1 : sb0;
    StreamBuf &nxt = P ? sb0 : sb1;
    const int kc0 = ci * kSK;
    const int nk_c = kv_rows(cu.nk - kc0);
    const bool last = kc0 + kSK >= cu.nk;
    if (!last) {
      dma_kv(nxt, cu, kc0 + kSK, kv_rows(cu.nk - kc0 - kSK));
    } else if (un < u_end) {
      // a one-chunk unit read its queries just now: every wave must be done
      // with the staging area before the next unit's copy lands there
      if (ci == 0) __syncthreads();
      dma_q(nu);
      dma_kv(nxt, nu, 0, kv_rows(nu.nk));
    }
    const int k0 = wave * 32;
    if (k0 < nk_c) {
      f32x16 sacc;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sacc[rr] = 0.f;
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const int kr = k0 + j;
        const u32x4 kraw = *reinterpret_cast<const u32x4 *>(
            &cur.Ks[kr * D + dkswz(kr, cc * 2 + h) * 8]);
        sacc = mfma32(as_bf16x8(kraw), qf[cc], sacc);
      }
      float x[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int key = k0 + 8 * (rr >> 2) + 4 * h + (rr & 3);
        x[rr] = key < nk_c ? sacc[rr] * scale_log2 : -INFINITY;
      }
      float mloc = x[0];
#pragma unroll
      for (int rr = 1; rr < 16; ++rr) mloc = fmaxf(mloc, x[rr]);
      // lazy rescale: the reference max moves only when the row max passes it
      // by more than 8, so every weight is at most 2^8
      const float mt = fmaxf(m, max_with_partner(mloc));   // finite: key k0 is valid
      if (__ballot(mt > m + kDecLazy)) {
        const float alpha = fast_exp2(m - mt);
        l *= alpha;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) acc[cb][rr] *= alpha;
        m = mt;
      }
      f32x8 p0, p1;
      float ps = 0.f;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        p0[rr] = fast_exp2(x[rr] - m);
        p1[rr] = fast_exp2(x[rr + 8] - m);
        ps += p0[rr] + p1[rr];
      }
      l += sum_with_partner(ps);
      const bf16x8 pb0 = __builtin_convertvector(p0, bf16x8);
      const bf16x8 pb1 = __builtin_convertvector(p1, bf16x8);
      const char *vbase = reinterpret_cast<const char *>(cur.Vs);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          constexpr int kRow = D * 2;
          const int o0 = voff[cb] + 16 * ks * kRow;
          const u32x2 lo = lds_read_tr(reinterpret_cast<const uint16_t *>(vbase + o0));
          const u32x2 hi = lds_read_tr(reinterpret_cast<const uint16_t *>(vbase + o0 + 8 * kRow));
          const u32x4 vraw = {lo[0], lo[1], hi[0], hi[1]};
          acc[cb] = mfma32(as_bf16x8(vraw), ks == 0 ? pb0 : pb1, acc[cb]);
        }
    }
    const uint32_t sg_cur = (uint32_t)cu.s * (uint32_t)hkv + (uint32_t)cu.g;
    if (last && (un >= u_end || (uint32_t)nu.s * (uint32_t)hkv + (uint32_t)nu.g != sg_cur)) {
      // the run ends: combine the four waves through LDS (the consumed
      // buffer), then store the run's partial before the chunk barrier's wait
      __syncthreads();
      float *mo = reinterpret_cast<float *>(&cur);   // [4][G][D]
      float *mm = mo + 4 * G * D;                    // [4][G]
      float *ml = mm + 4 * G;                        // [4][G]
      if (j < G) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg)
            *reinterpret_cast<float4 *>(&mo[(wave * G + j) * D + cb * 32 + 8 * rg + 4 * h]) =
                make_float4(acc[cb][4 * rg], acc[cb][4 * rg + 1], acc[cb][4 * rg + 2],
                            acc[cb][4 * rg + 3]);
        if (h == 0) {
          mm[wave * G + j] = m;
          ml[wave * G + j] = l;
        }
      }
      __syncthreads();
      const size_t sl = run_slot(sg_cur);
      if constexpr (FUSED) {
        // four consecutive columns per thread, stored device-coherent
        const __amdgpu_buffer_rsrc_t ro = record_rsrc(part_o + sl * G * D, G * D * 4);
        const __amdgpu_buffer_rsrc_t rl = record_rsrc(part_lse + sl * G, G * 4);
        for (int x4 = tid; x4 < G * D / 4; x4 += 256) {
          const int hd = x4 / (D / 4), c4 = (x4 % (D / 4)) * 4;
          float mx = -INFINITY;
#pragma unroll
          for (int w = 0; w < 4; ++w) mx = fmaxf(mx, mm[w * G + hd]);
          float z = 0.f;
          float ov[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float sc = fast_exp2(mm[w * G + hd] - mx);   // 0 for a wave without keys
            z = fmaf(sc, ml[w * G + hd], z);
            const float4 m4 = *reinterpret_cast<const float4 *>(&mo[(w * G + hd) * D + c4]);
            ov[0] = fmaf(sc, m4.x, ov[0]);
            ov[1] = fmaf(sc, m4.y, ov[1]);
            ov[2] = fmaf(sc, m4.z, ov[2]);
            ov[3] = fmaf(sc, m4.w, ov[3]);
          }
          store_sc1(ro, (hd * D + c4) * 4, make_float4(ov[0] / z, ov[1] / z, ov[2] / z, ov[3] / z));
          if (c4 == 0) store_sc1(rl, hd * 4, mx + __log2f(z));
        }
      } else {
        for (int x = tid; x < G * D; x += 256) {
          const int hd = x / D, c = x % D;
          float mx = -INFINITY;
#pragma unroll
          for (int w = 0; w < 4; ++w) mx = fmaxf(mx, mm[w * G + hd]);
          float z = 0.f, ov = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float sc = fast_exp2(mm[w * G + hd] - mx);   // 0 for a wave without keys
            z = fmaf(sc, ml[w * G + hd], z);
            ov = fmaf(sc, mo[(w * G + hd) * D + c], ov);
          }
          part_o[(sl * G + hd) * D + c] = ov / z;
          if (c == 0) part_lse[sl * G + hd] = mx + __log2f(z);
        }
      }
      arrive(sg_cur);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // One unit whose first chunk sits in buffer P0; returns the buffer of the
  // next unit's first chunk, or -1 when the range is done.
  auto run_unit = [&](auto ptag) __attribute__((always_inline)) -> int {
    constexpr int P0 = decltype(ptag)::value;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      u32x4 xq = *reinterpret_cast<const u32x4 *>(&qs[(j < G ? j : 0) * D + cc * 16 + 8 * h]);
      if (j >= G) xq = u32x4{0u, 0u, 0u, 0u};
      qf[cc] = as_bf16x8(xq);
    }
    // the staging area is rewritten by the next unit's DMA: finish these reads
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), others untouched
    const uint32_t sg = (uint32_t)cu.s * (uint32_t)hkv + (uint32_t)cu.g;
    if (sg >= sg_next) {   // a new run (runs whose units were all empty: neutral)
      for (; sg_next < sg; ++sg_next) put_neutral(sg_next);
      sg_next = sg + 1;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) acc[cb][rr] = 0.f;
      m = -INFINITY;
      l = 0.f;
    }
    ci = 0;
    int endp;
    for (;;) {
      chunk(std::integral_constant<int, P0>{});
      if ((ci + 1) * kSK >= cu.nk) { endp = P0; break; }
      ++ci;
      chunk(std::integral_constant<int, 1 - P0>{});
      if ((ci + 1) * kSK >= cu.nk) { endp = 1 - P0; break; }
      ++ci;
    }
    if (un >= u_end) return -1;
    u = un;
    cu = nu;
    un = next_unit(u + 1, nu);
    return 1 - endp;
  };

  int par = 0;
  for (;;) {
    const int nx = par ? run_unit(std::integral_constant<int, 1>{})
                       : run_unit(std::integral_constant<int, 0>{});
    if (nx < 0) break;
    par = nx;
  }
  for (; sg_next <= (u_end - 1) / ups_g; ++sg_next) put_neutral(sg_next);
}

// ---------------------------------------------------------------------------
// Paged KV cache, bf16 or FP8 (e4m3) keys and values: the decode attention of
// decode_stream over a page pool.  A page holds one MSA block of one KV head
// ([n_pages][Hkv][B][d]); logical block b of sequence s lives in page
// block_table[s][b].  FP8 pages carry one scale per (page, KV head) for K and
// one for V: k = k_scale * e4m3(k_page), likewise v.  The units and the chunk
// stream are those of decode_stream (non-fused).  bf16 pages also keep its
// runs (one partial per run); an FP8 unit never leaves its block, so its two
// scales are constants: the scores are scaled once (folded into the softmax
// scale) and the partial output once at the unit's end -- one partial per
// unit.
//
// decode_paged is the bf16 kernel (decode_stream's double-buffered chunk
// stream with page addressing); decode_paged_fp8 below the FP8 one.
// ---------------------------------------------------------------------------
template <bool FP8>
struct PagedBuf;
template <>
struct PagedBuf<false> {
  uint16_t Ks[kSK * 128];
  uint16_t Vs[kSK * 128];
};
template <>
struct PagedBuf<true> {
  uint8_t Ks[kSK * 128];
  uint8_t Vs[kSK * 128];
};

struct PagedUnit {
  int s, g;
  int64_t row0;    // element offset of the unit's first key row in the page pool
  int nk;          // keys in the unit (0: empty)
  float ks, vs;    // the page's K and V scales (1 for bf16)
};
constexpr int kUnitTab = 64;   // units per workgroup resolved up front

// 8 e4m3 bytes -> 8 bf16 (exact: every e4m3 value is a bf16 value)
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return u32x4{
      __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false)),
      __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true)),
      __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false)),
      __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true))};
}

template <int G>
__global__ __launch_bounds__(256) void decode_paged(
    const uint16_t *__restrict__ q, const uint8_t *__restrict__ kpool,
    const uint8_t *__restrict__ vpool, const float *__restrict__ k_scale,
    const float *__restrict__ v_scale, const int32_t *__restrict__ block_table,
    int max_blocks, int64_t n_pages, const int64_t *__restrict__ seq_len, int hq, int hkv,
    int B, const int32_t *__restrict__ sel, int topk, int nseg, int seg_len, uint32_t u_q,
    uint32_t u_r, float scale_log2, float *__restrict__ part_o,
    float *__restrict__ part_lse) {
  constexpr int D = 128;
  constexpr int RB = D * 2;                       // bytes per row
  constexpr int SPR = RB / 16;                    // 16-byte slots per row
  constexpr int IPW = (kSK * SPR) / 256;          // DMA instructions per wave per tensor
  constexpr int QE = G * D < 512 ? 512 : G * D;   // staged query elements
  __shared__ PagedBuf<false> sb0;
  __shared__ PagedBuf<false> sb1;
  __shared__ uint16_t qs[QE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, j = lane & 31;
  const int64_t len_max = (int64_t)max_blocks * B;

  const uint32_t bx = blockIdx.x;
  const uint32_t u_begin = bx * u_q + (bx < u_r ? bx : u_r);
  const uint32_t u_end = u_begin + u_q + (bx < u_r ? 1u : 0u);

  auto unit = [&](uint32_t u) __attribute__((always_inline)) {
    PagedUnit d;
    // decode_stream's unit order (segment-major, the row's last entry first),
    // so both kernels accumulate a run's units in the same order
    const uint32_t upg = (uint32_t)(topk * nseg);
    const uint32_t sgi = u / upg, idx = u - sgi * upg;
    const int seg = (int)(idx / (uint32_t)topk);
    const int kr = (int)(idx - (uint32_t)seg * (uint32_t)topk);
    const int kk = kr == 0 ? topk - 1 : kr - 1;
    d.s = (int)(sgi / (uint32_t)hkv);
    d.g = (int)(sgi - (uint32_t)d.s * (uint32_t)hkv);
    int64_t len = seq_len[d.s];
    if (len > len_max) len = len_max;
    const int32_t b = sel[(int64_t)d.s * topk + kk];
    const int32_t page =
        (b >= 0 && b < max_blocks) ? block_table[(int64_t)d.s * max_blocks + b] : -1;
    const int64_t t0 = (int64_t)b * B + (int64_t)seg * seg_len;
    int64_t n = (page < 0 || page >= n_pages || len < 1) ? 0 : len - t0;   // keys t0 .. len-1
    if (n > seg_len) n = seg_len;
    if (n > (int64_t)B - (int64_t)seg * seg_len) n = (int64_t)B - (int64_t)seg * seg_len;
    d.nk = n > 0 ? (int)n : 0;
    d.row0 = d.nk > 0 ? ((int64_t)page * hkv + d.g) * B + (int64_t)seg * seg_len : 0;
    d.ks = 1.f;
    d.vs = 1.f;
    return d;
  };
  // The range's first kUnitTab units, resolved once at the start by one
  // thread each, so their dependent loads (selection -> block table ->
  // scales) are in flight together instead of stalling the copy cursor at
  // every unit boundary; later units are resolved when reached.
  __shared__ PagedUnit utab[kUnitTab];
  {
    const uint32_t n_tab = u_end - u_begin < (uint32_t)kUnitTab ? u_end - u_begin : kUnitTab;
    for (uint32_t t = tid; t < n_tab; t += 256) utab[t] = unit(u_begin + t);
    __syncthreads();
  }
  auto unit_c = [&](uint32_t u) __attribute__((always_inline)) {
    return u - u_begin < (uint32_t)kUnitTab ? utab[u - u_begin] : unit(u);
  };
  auto next_unit = [&](uint32_t u, PagedUnit &d) __attribute__((always_inline)) {
    for (; u < u_end; ++u) {
      d = unit_c(u);
      if (d.nk > 0) break;
    }
    return u;
  };
  // runs of one (sequence, KV head), as in decode_stream (bf16 pages: no V
  // scale, so a run may cross pages)
  const uint32_t ups_g = (uint32_t)(topk * nseg);
  auto run_slot = [&](uint32_t sg) __attribute__((always_inline)) {
    const uint32_t u0 = sg * ups_g;
    return u0 > u_begin ? u0 : u_begin;
  };
  auto put_neutral = [&](uint32_t sg) __attribute__((always_inline)) {
    const size_t sl = run_slot(sg);
    for (int x = tid; x < G * D; x += 256) part_o[sl * G * D + x] = 0.f;
    if (tid < G) part_lse[sl * G + tid] = -INFINITY;
  };
  uint32_t sg_next = u_begin / ups_g;
  // K and V rows with decode_stream's swizzles
  auto dma_kv = [&](PagedBuf<false> &buf, const PagedUnit &d, int64_t row, int nrows)
      __attribute__((always_inline)) {
    const uint8_t *kb = kpool + (d.row0 + row) * RB;
    const uint8_t *vb = vpool + (d.row0 + row) * RB;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int inst = wave * IPW + i;
      const int pslot = inst * 64 + lane;
      const int r = pslot / SPR, sp = pslot % SPR;
      const int64_t rr = r < nrows ? r : nrows - 1;   // rows past the end repeat the last
      const int ksl = dkswz(r, sp);
      const int vsl = dvswz(r, sp);
      __builtin_amdgcn_global_load_lds(
          (dec_gptr_t)(const_cast<uint8_t *>(kb + rr * RB + ksl * 16)),
          (dec_lptr_t)(reinterpret_cast<uint8_t *>(buf.Ks) + inst * 64 * 16), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          (dec_gptr_t)(const_cast<uint8_t *>(vb + rr * RB + vsl * 16)),
          (dec_lptr_t)(reinterpret_cast<uint8_t *>(buf.Vs) + inst * 64 * 16), 16, 0, 0);
    }
  };
  auto dma_q = [&](const PagedUnit &d) __attribute__((always_inline)) {
    if (wave == 0) {
      const uint16_t *qb = q + ((int64_t)d.s * hq + (int64_t)d.g * G) * D;
#pragma unroll
      for (int i = 0; i < QE / 512; ++i) {
        const int off = (i * 512 + lane * 8) % (G * D);
        __builtin_amdgcn_global_load_lds((dec_gptr_t)(const_cast<uint16_t *>(qb + off)),
                                         (dec_lptr_t)(&qs[i * 512]), 16, 0, 0);
      }
    }
  };
  auto kv_rows = [&](int n) __attribute__((always_inline)) { return n < kSK ? n : kSK; };

  PagedUnit cu;
  uint32_t u = next_unit(u_begin, cu);
  if (u >= u_end) {
    for (uint32_t sg = sg_next; sg <= (u_end - 1) / ups_g; ++sg) put_neutral(sg);
    return;
  }
  PagedUnit nu = cu;
  uint32_t un = next_unit(u + 1, nu);
  dma_q(cu);
  dma_kv(sb0, cu, 0, kv_rows(cu.nk));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  int voff[4];
  {
    const int a16 = lane & 15;
    const int vrow = wave * 32 + 4 * h + (a16 >> 2);
    const int vcol0 = 16 * (j >> 4) + 4 * (a16 & 3);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int col = cb * 32 + vcol0;
      voff[cb] = (vrow * D + dvswz(vrow, col >> 3) * 8 + (col & 7)) * 2;
    }
  }

  bf16x8 qf[8];
  f32x16 acc[4];
  float m = -INFINITY, l = 0.f;
  int ci = 0;

  auto chunk = [&](auto tag) __attribute__((always_inline)) {
    constexpr int P = decltype(tag)::value;
    PagedBuf<false> &cur = P ? sb1 : sb0;
    PagedBuf<false> &nxt = P ? sb0 : sb1;
    const int kc0 = ci * kSK;
    const int nk_c = kv_rows(cu.nk - kc0);
    const bool last = kc0 + kSK >= cu.nk;
    if (!last) {
      dma_kv(nxt, cu, kc0 + kSK, kv_rows(cu.nk - kc0 - kSK));
    } else if (un < u_end) {
      if (ci == 0) __syncthreads();   // every wave has read this unit's queries
      dma_q(nu);
      dma_kv(nxt, nu, 0, kv_rows(nu.nk));
    }
    const int k0 = wave * 32;
    if (k0 < nk_c) {
      f32x16 sacc;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sacc[rr] = 0.f;
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const int kr = k0 + j;
        const u32x4 kraw =
            *reinterpret_cast<const u32x4 *>(&cur.Ks[kr * D + dkswz(kr, cc * 2 + h) * 8]);
        sacc = mfma32(as_bf16x8(kraw), qf[cc], sacc);
      }
      const float sl = scale_log2 * cu.ks;
      float x[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int key = k0 + 8 * (rr >> 2) + 4 * h + (rr & 3);
        x[rr] = key < nk_c ? sacc[rr] * sl : -INFINITY;
      }
      float mloc = x[0];
#pragma unroll
      for (int rr = 1; rr < 16; ++rr) mloc = fmaxf(mloc, x[rr]);
      // lazy rescale: the reference max moves only when the row max passes it
      // by more than 8, so every weight is at most 2^8
      const float mt = fmaxf(m, max_with_partner(mloc));
      if (__ballot(mt > m + kDecLazy)) {
        const float alpha = fast_exp2(m - mt);
        l *= alpha;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) acc[cb][rr] *= alpha;
        m = mt;
      }
      f32x8 p0, p1;
      float ps = 0.f;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        p0[rr] = fast_exp2(x[rr] - m);
        p1[rr] = fast_exp2(x[rr + 8] - m);
        ps += p0[rr] + p1[rr];
      }
      l += sum_with_partner(ps);
      const bf16x8 pb0 = __builtin_convertvector(p0, bf16x8);
      const bf16x8 pb1 = __builtin_convertvector(p1, bf16x8);
      const char *vbase = reinterpret_cast<const char *>(cur.Vs);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          constexpr int kRow = D * 2;
          const int o0 = voff[cb] + 16 * ks * kRow;
          const u32x2 lo = lds_read_tr(reinterpret_cast<const uint16_t *>(vbase + o0));
          const u32x2 hi = lds_read_tr(reinterpret_cast<const uint16_t *>(vbase + o0 + 8 * kRow));
          const u32x4 vraw = {lo[0], lo[1], hi[0], hi[1]};
          acc[cb] = mfma32(as_bf16x8(vraw), ks == 0 ? pb0 : pb1, acc[cb]);
        }
    }
    const uint32_t sg_cur = (uint32_t)cu.s * (uint32_t)hkv + (uint32_t)cu.g;
    if (last && (un >= u_end || (uint32_t)nu.s * (uint32_t)hkv + (uint32_t)nu.g != sg_cur)) {
      __syncthreads();
      // the waves' (o, m, l) through LDS, in the consumed chunk buffer
      static_assert(4 * G * D * 4 + 8 * G * 4 <= (int)sizeof(PagedBuf<false>), "");
      float *mo = reinterpret_cast<float *>(&cur);   // [4][G][D]
      float *mm = mo + 4 * G * D;                    // [4][G]
      float *ml = mm + 4 * G;                        // [4][G]
      if (j < G) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg)
            *reinterpret_cast<float4 *>(&mo[(wave * G + j) * D + cb * 32 + 8 * rg + 4 * h]) =
                make_float4(acc[cb][4 * rg], acc[cb][4 * rg + 1], acc[cb][4 * rg + 2],
                            acc[cb][4 * rg + 3]);
        if (h == 0) {
          mm[wave * G + j] = m;
          ml[wave * G + j] = l;
        }
      }
      __syncthreads();
      for (int x = tid; x < G * D; x += 256) {
        const int hd = x / D, c = x % D;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) mx = fmaxf(mx, mm[w * G + hd]);
        float z = 0.f, ov = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float sc = fast_exp2(mm[w * G + hd] - mx);
          z = fmaf(sc, ml[w * G + hd], z);
          ov = fmaf(sc, mo[(w * G + hd) * D + c], ov);
        }
        const size_t sl = run_slot(sg_cur);
        part_o[(sl * G + hd) * D + c] = ov / z;
        if (c == 0) part_lse[sl * G + hd] = mx + __log2f(z);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  auto run_unit = [&](auto ptag) __attribute__((always_inline)) -> int {
    constexpr int P0 = decltype(ptag)::value;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      u32x4 xq = *reinterpret_cast<const u32x4 *>(&qs[(j < G ? j : 0) * D + cc * 16 + 8 * h]);
      if (j >= G) xq = u32x4{0u, 0u, 0u, 0u};
      qf[cc] = as_bf16x8(xq);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    const uint32_t sg = (uint32_t)cu.s * (uint32_t)hkv + (uint32_t)cu.g;
    if (sg >= sg_next) {   // a new run (runs whose units were all empty: neutral)
      for (; sg_next < sg; ++sg_next) put_neutral(sg_next);
      sg_next = sg + 1;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) acc[cb][rr] = 0.f;
      m = -INFINITY;
      l = 0.f;
    }
    ci = 0;
    int endp;
    for (;;) {
      chunk(std::integral_constant<int, P0>{});
      if ((ci + 1) * kSK >= cu.nk) { endp = P0; break; }
      ++ci;
      chunk(std::integral_constant<int, 1 - P0>{});
      if ((ci + 1) * kSK >= cu.nk) { endp = 1 - P0; break; }
      ++ci;
    }
    if (un >= u_end) return -1;
    u = un;
    cu = nu;
    un = next_unit(u + 1, nu);
    return 1 - endp;
  };

  int par = 0;
  for (;;) {
    const int nx = par ? run_unit(std::integral_constant<int, 1>{})
                       : run_unit(std::integral_constant<int, 0>{});
    if (nx < 0) break;
    par = nx;
  }
  for (; sg_next <= (u_end - 1) / ups_g; ++sg_next) put_neutral(sg_next);
}

// ---------------------------------------------------------------------------
// FP8 pages, three chunk buffers.  An FP8 chunk of 128 keys is half the bytes
// of a bf16 one; three 32 KiB buffers keep two chunks in flight while the
// third is computed.  K is widened to bf16 in registers as in decode_paged;
// V^T operands come straight from the FP8 rows by ds_read_b64_tr_b8 (a
// 16-lane group reads 8 keys x 16 columns and each lane receives its
// column's 8 keys, exactly one bf16 MFMA operand after widening), so no
// staging pass is needed.  The copies and
// waits are written out (inline assembly) rather than left to the compiler,
// which cannot always tell a copy into one buffer from reads of another and
// then waits for every copy in flight: each wave waits until at most the
// loads of chunk i+2 are outstanding (loads complete in order), then a
// fence-free barrier publishes chunk i+1.  Units, scaling and partials as
// decode_paged.
// ---------------------------------------------------------------------------
// 16 bytes per lane from global memory straight into LDS at lds_base + 16 *
// lane (lds_base is wave-uniform and goes through M0).  No register receives
// data, so nothing is live while the copy is in flight.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// LDS-visibility barrier without a memory fence: loads in flight stay so.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// LDS offset of a shared-memory object (its local address-space pointer).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(dec_lptr_t)(const_cast<void *>(p));
}
// Transposed 8-bit read: within each 16-lane group, lane i supplies the
// address of 8 bytes (row i/2, half i%2 of a 16-byte column span) and
// receives column i's bytes from the group's 8 rows.
typedef int dec_i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) dec_i32x2 *dec_lds_i32x2_ptr;
__device__ __forceinline__ u32x2 lds_read_tr8(const uint8_t *p) {
  const dec_i32x2 r =
      __builtin_amdgcn_ds_read_tr8_b64_v2i32((dec_lds_i32x2_ptr)(const_cast<uint8_t *>(p)));
  return __builtin_bit_cast(u32x2, r);
}

template <int G>
__global__ __launch_bounds__(256) void decode_paged_fp8(
    const uint16_t *__restrict__ q, const uint8_t *__restrict__ kpool,
    const uint8_t *__restrict__ vpool, const float *__restrict__ k_scale,
    const float *__restrict__ v_scale, const int32_t *__restrict__ block_table,
    int max_blocks, int64_t n_pages, const int64_t *__restrict__ seq_len, int hq, int hkv,
    int B, const int32_t *__restrict__ sel, int topk, int nseg, int seg_len, uint32_t u_q,
    uint32_t u_r, float scale_log2, float *__restrict__ part_o,
    float *__restrict__ part_lse) {
  constexpr int D = 128;
  constexpr int RB = D;                           // bytes per FP8 row
  constexpr int SPR = RB / 16;                    // 16-byte slots per row
  constexpr int IPW = (kSK * SPR) / 256;          // copy instructions per wave per tensor
  constexpr int kChunkOps = 2 * IPW;              // loads per wave per chunk
  constexpr int QE = G * D < 512 ? 512 : G * D;
  static_assert(kChunkOps < 16, "vmcnt immediate");
  static_assert(4 * G * D * 4 <= (int)sizeof(PagedBuf<true>), "combine fits a buffer");
  __shared__ PagedBuf<true> sb0;
  __shared__ PagedBuf<true> sb1;
  __shared__ PagedBuf<true> sb2;
  __shared__ uint16_t qs[QE];
  __shared__ float mml[2 * 4 * G];   // the waves' (max, sum) at a unit's end
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, j = lane & 31;
  const int64_t len_max = (int64_t)max_blocks * B;

  const uint32_t bx = blockIdx.x;
  const uint32_t u_begin = bx * u_q + (bx < u_r ? bx : u_r);
  const uint32_t u_end = u_begin + u_q + (bx < u_r ? 1u : 0u);

  auto unit = [&](uint32_t u) __attribute__((always_inline)) {
    PagedUnit d;
    const uint32_t r1 = u / (uint32_t)nseg;
    const int seg = (int)(u - r1 * (uint32_t)nseg);
    const uint32_t r2 = r1 / (uint32_t)topk;
    const int kk = (int)(r1 - r2 * (uint32_t)topk);
    const uint32_t r3 = r2 / (uint32_t)hkv;
    d.g = (int)(r2 - r3 * (uint32_t)hkv);
    d.s = (int)r3;
    int64_t len = seq_len[d.s];
    if (len > len_max) len = len_max;
    const int32_t b = sel[(int64_t)d.s * topk + kk];
    const int32_t page =
        (b >= 0 && b < max_blocks) ? block_table[(int64_t)d.s * max_blocks + b] : -1;
    const int64_t t0 = (int64_t)b * B + (int64_t)seg * seg_len;
    int64_t n = (page < 0 || page >= n_pages || len < 1) ? 0 : len - t0;
    if (n > seg_len) n = seg_len;
    if (n > (int64_t)B - (int64_t)seg * seg_len) n = (int64_t)B - (int64_t)seg * seg_len;
    d.nk = n > 0 ? (int)n : 0;
    d.row0 = d.nk > 0 ? ((int64_t)page * hkv + d.g) * B + (int64_t)seg * seg_len : 0;
    d.ks = d.nk > 0 ? k_scale[(int64_t)page * hkv + d.g] : 1.f;
    d.vs = d.nk > 0 ? v_scale[(int64_t)page * hkv + d.g] : 1.f;
    return d;
  };
  // The range's first kUnitTab units, resolved once at the start by one
  // thread each, so their dependent loads (selection -> block table ->
  // scales) are in flight together instead of stalling the copy cursor at
  // every unit boundary; later units are resolved when reached.
  __shared__ PagedUnit utab[kUnitTab];
  {
    const uint32_t n_tab = u_end - u_begin < (uint32_t)kUnitTab ? u_end - u_begin : kUnitTab;
    for (uint32_t t = tid; t < n_tab; t += 256) utab[t] = unit(u_begin + t);
    __syncthreads();
  }
  auto unit_c = [&](uint32_t u) __attribute__((always_inline)) {
    return u - u_begin < (uint32_t)kUnitTab ? utab[u - u_begin] : unit(u);
  };
  auto next_unit = [&](uint32_t u, PagedUnit &d) __attribute__((always_inline)) {
    for (; u < u_end; ++u) {
      d = unit_c(u);
      if (d.nk > 0) break;
    }
    return u;
  };
  // Runs of one (sequence, KV head), as in decode_paged: the page's V scale
  // is folded into the weights of its keys (the normaliser keeps the
  // unscaled ones), so the online softmax runs on across pages and one
  // partial per run is written, in the slot of the run's first unit in this
  // workgroup's range; a run whose units are all empty gets the neutral one.
  const uint32_t ups_g = (uint32_t)(topk * nseg);
  auto run_slot = [&](uint32_t sg) __attribute__((always_inline)) {
    const uint32_t u0 = sg * ups_g;
    return u0 > u_begin ? u0 : u_begin;
  };
  auto put_neutral = [&](uint32_t sg) __attribute__((always_inline)) {
    const size_t sl = run_slot(sg);
    for (int x = tid; x < G * D; x += 256) part_o[sl * G * D + x] = 0.f;
    if (tid < G) part_lse[sl * G + tid] = -INFINITY;
  };
  uint32_t sg_next = u_begin / ups_g;
  auto dma_kv = [&](PagedBuf<true> &buf, const PagedUnit &d, int64_t row, int nrows)
      __attribute__((always_inline)) {
    const uint8_t *kb = kpool + (d.row0 + row) * RB;
    const uint8_t *vb = vpool + (d.row0 + row) * RB;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int inst = wave * IPW + i;
      const int pslot = inst * 64 + lane;
      const int r = pslot / SPR, sp = pslot % SPR;
      const int64_t rr = r < nrows ? r : nrows - 1;
      dma16(kb + rr * RB + (sp ^ (r & 7)) * 16, lds_addr(&buf.Ks[inst * 64 * 16]));
      dma16(vb + rr * RB + (sp ^ (r & 7)) * 16, lds_addr(&buf.Vs[inst * 64 * 16]));
    }
  };
  auto dma_q = [&](const PagedUnit &d) __attribute__((always_inline)) {
    if (wave == 0) {
      const uint16_t *qb = q + ((int64_t)d.s * hq + (int64_t)d.g * G) * D;
#pragma unroll
      for (int i = 0; i < QE / 512; ++i) {
        const int off = (i * 512 + lane * 8) % (G * D);
        dma16(qb + off, lds_addr(&qs[i * 512]));
      }
    }
  };
  auto kv_rows = [&](int n) __attribute__((always_inline)) { return n < kSK ? n : kSK; };

  // compute cursor (unit u, chunk ci) and the next non-empty unit
  PagedUnit cu;
  uint32_t u = next_unit(u_begin, cu);
  if (u >= u_end) {
    for (uint32_t sg = sg_next; sg <= (u_end - 1) / ups_g; ++sg) put_neutral(sg);
    return;
  }
  PagedUnit nu = cu;
  uint32_t un = next_unit(u + 1, nu);
  // copy cursor, two chunks ahead
  PagedUnit du = cu;
  uint32_t ud = u;
  int cd = 0;
  auto dma_item = [&](PagedBuf<true> &buf) __attribute__((always_inline)) -> bool {
    if (ud >= u_end) return false;
    dma_kv(buf, du, (int64_t)cd * kSK, kv_rows(du.nk - cd * kSK));
    if (++cd * kSK >= du.nk) {
      ud = next_unit(ud + 1, du);
      cd = 0;
    }
    return true;
  };

  dma_q(cu);
  dma_item(sb0);
  if (dma_item(sb1))
    wait_vm<kChunkOps>();   // the queries and chunk 0 landed
  else
    wait_vm<0>();
  lds_barrier();

  // V^T operand offsets (bytes), per column block: lane a16 of a 16-lane
  // group supplies the group's key a16/2 and the 8-byte half a16%2 of its 16
  // columns; rows keep their 16-byte slots XOR-swizzled by row.  The 8 keys
  // of a lane's operand follow the score tile's row order (keys 4h .. 4h+3
  // and 8+4h .. 8+4h+3 of the 16-key step), which the probabilities share.
  int voff[4];
  {
    const int a16 = lane & 15, ri = a16 >> 1;
    const int vrow = wave * 32 + 8 * (ri >> 2) + 4 * h + (ri & 3);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int slot = 2 * cb + (j >> 4);
      voff[cb] = vrow * RB + ((slot ^ (vrow & 7)) << 4) + ((a16 & 1) << 3);
    }
  }

  bf16x8 qf[8];
  f32x16 acc[4];
  float m = -INFINITY, l = 0.f;
  int ci = 0;

  auto step = [&](auto tag) __attribute__((always_inline)) -> bool {
    constexpr int P = decltype(tag)::value;
    PagedBuf<true> &cur = P == 0 ? sb0 : (P == 1 ? sb1 : sb2);
    PagedBuf<true> &far = P == 0 ? sb2 : (P == 1 ? sb0 : sb1);   // chunk i+2
    if (ci == 0) {
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        u32x4 xq = *reinterpret_cast<const u32x4 *>(&qs[(j < G ? j : 0) * D + cc * 16 + 8 * h]);
        if (j >= G) xq = u32x4{0u, 0u, 0u, 0u};
        qf[cc] = as_bf16x8(xq);
      }
      const uint32_t sg = (uint32_t)cu.s * (uint32_t)hkv + (uint32_t)cu.g;
      if (sg >= sg_next) {   // a new run (runs whose units were all empty: neutral)
        for (; sg_next < sg; ++sg_next) put_neutral(sg_next);
        sg_next = sg + 1;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) acc[cb][rr] = 0.f;
        m = -INFINITY;
        l = 0.f;
      }
      if (un < u_end) {
        lds_barrier();   // every wave holds its queries: the staging area is free
        dma_q(nu);
      }
    }
    const bool has2 = dma_item(far);
    const int kc0 = ci * kSK;
    const int nk_c = kv_rows(cu.nk - kc0);
    const bool last = kc0 + kSK >= cu.nk;
    const int k0 = wave * 32;
    if (k0 < nk_c) {
      f32x16 sacc;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sacc[rr] = 0.f;
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const int kr = k0 + j;
        const u32x2 r8 = *reinterpret_cast<const u32x2 *>(
            &cur.Ks[kr * RB + ((cc ^ (kr & 7)) * 16) + 8 * h]);
        sacc = mfma32(as_bf16x8(fp8x8_to_bf16x8(r8[0], r8[1])), qf[cc], sacc);
      }
      const float sl = scale_log2 * cu.ks;
      float x[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int key = k0 + 8 * (rr >> 2) + 4 * h + (rr & 3);
        x[rr] = key < nk_c ? sacc[rr] * sl : -INFINITY;
      }
      float mloc = x[0];
#pragma unroll
      for (int rr = 1; rr < 16; ++rr) mloc = fmaxf(mloc, x[rr]);
      // lazy rescale: the reference max moves only when the row max passes it
      // by more than 8, so every weight is at most 2^8
      const float mt = fmaxf(m, max_with_partner(mloc));
      if (__ballot(mt > m + kDecLazy)) {
        const float alpha = fast_exp2(m - mt);
        l *= alpha;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) acc[cb][rr] *= alpha;
        m = mt;
      }
      f32x8 p0, p1;
      float ps = 0.f;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        p0[rr] = fast_exp2(x[rr] - m);
        p1[rr] = fast_exp2(x[rr + 8] - m);
        ps += p0[rr] + p1[rr];
      }
      l += sum_with_partner(ps);
      // the P.V weights carry the page's V scale
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        p0[rr] *= cu.vs;
        p1[rr] *= cu.vs;
      }
      const bf16x8 pb0 = __builtin_convertvector(p0, bf16x8);
      const bf16x8 pb1 = __builtin_convertvector(p1, bf16x8);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const u32x2 v8 = lds_read_tr8(&cur.Vs[voff[cb] + 16 * ks * RB]);
          acc[cb] = mfma32(as_bf16x8(fp8x8_to_bf16x8(v8[0], v8[1])), ks == 0 ? pb0 : pb1,
                           acc[cb]);
        }
    }
    // chunk i+1 (and the next unit's queries, copied before chunk i+2) landed
    if (has2)
      wait_vm<kChunkOps>();
    else
      wait_vm<0>();
    const uint32_t sg_cur = (uint32_t)cu.s * (uint32_t)hkv + (uint32_t)cu.g;
    if (last && (un >= u_end || (uint32_t)nu.s * (uint32_t)hkv + (uint32_t)nu.g != sg_cur)) {
      lds_barrier();
      float *mo = reinterpret_cast<float *>(&cur);      // [4][G][D]
      float *mm = mml;                                  // [4][G]
      float *ml = mml + 4 * G;                          // [4][G]
      if (j < G) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg)
            *reinterpret_cast<float4 *>(&mo[(wave * G + j) * D + cb * 32 + 8 * rg + 4 * h]) =
                make_float4(acc[cb][4 * rg], acc[cb][4 * rg + 1], acc[cb][4 * rg + 2],
                            acc[cb][4 * rg + 3]);
        if (h == 0) {
          mm[wave * G + j] = m;
          ml[wave * G + j] = l;
        }
      }
      lds_barrier();
      for (int x = tid; x < G * D; x += 256) {
        const int hd = x / D, c = x % D;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) mx = fmaxf(mx, mm[w * G + hd]);
        float z = 0.f, ov = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float sc = fast_exp2(mm[w * G + hd] - mx);
          z = fmaf(sc, ml[w * G + hd], z);
          ov = fmaf(sc, mo[(w * G + hd) * D + c], ov);
        }
        const size_t sl = run_slot(sg_cur);
        part_o[(sl * G + hd) * D + c] = ov / z;
        if (c == 0) part_lse[sl * G + hd] = mx + __log2f(z);
      }
    }
    lds_barrier();   // chunk i+1 visible to every wave; buffer P reusable
    if (!last) {
      ++ci;
      return true;
    }
    if (un >= u_end) return false;
    u = un;
    cu = nu;
    un = next_unit(u + 1, nu);
    ci = 0;
    return true;
  };

  for (;;) {
    if (!step(std::integral_constant<int, 0>{})) break;
    if (!step(std::integral_constant<int, 1>{})) break;
    if (!step(std::integral_constant<int, 2>{})) break;
  }
  for (; sg_next <= (u_end - 1) / ups_g; ++sg_next) put_neutral(sg_next);
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
#pragma unroll 16
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

// Merge of decode_stream's run partials: the units of (sequence s, KV head
// g) are [sg * ups_g, (sg + 1) * ups_g) with sg = s * hkv + g; the
// workgroups whose static unit ranges (u_q each, one more for the first u_r)
// meet that span each left one partial, in the slot of their first unit in
// it.  Workgroup = (query head, sequence), one thread per column.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_runs(
    int G, int hkv, uint32_t ups_g, uint32_t u_q, uint32_t u_r,
    const float *__restrict__ part_o, const float *__restrict__ part_lse,
    float *__restrict__ o, float *__restrict__ lse) {
  const int hh = blockIdx.x, s = blockIdx.y, c = threadIdx.x;
  const int hq = gridDim.x, g = hh / G, hl = hh % G;
  const uint32_t sg = (uint32_t)s * (uint32_t)hkv + (uint32_t)g;
  const uint32_t u0 = sg * ups_g, u1 = u0 + ups_g - 1;
  const uint32_t split = u_r * (u_q + 1);   // units of the longer ranges
  auto wg_of = [&](uint32_t u) { return u < split ? u / (u_q + 1) : u_r + (u - split) / u_q; };
  const uint32_t b0 = wg_of(u0), b1 = wg_of(u1);
  float m = -3.0e38f, z = 0.f, acc = 0.f;
  constexpr int kBatch = 16;   // partials whose loads are in flight together
  for (uint32_t bx0 = b0; bx0 <= b1; bx0 += kBatch) {
    float li[kBatch], oi[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const uint32_t bx = bx0 + k;
      li[k] = -INFINITY;
      oi[k] = 0.f;
      if (bx <= b1) {
        const uint32_t ub = bx * u_q + (bx < u_r ? bx : u_r);
        const size_t sl = ub > u0 ? ub : u0;
        li[k] = part_lse[sl * G + hl];
        oi[k] = part_o[(sl * G + hl) * D + c];
      }
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float mn = fmaxf(m, li[k]);
      const float sc = fast_exp2(m - mn), w = fast_exp2(li[k] - mn);
      z = fmaf(z, sc, w);
      acc = fmaf(acc, sc, w * oi[k]);
      m = mn;
    }
  }
  o[((int64_t)s * hq + hh) * D + c] = acc / z;
  if (lse && c == 0) lse[(int64_t)s * hq + hh] = (m + __log2f(z)) * kLn2;
}

// ---------------------------------------------------------------------------
// Fused decode step, stage 1: workgroup = (chunk of kDecChunk blocks,
// sequence), plus one more workgroup per sequence (x = n_chunks) that appends
// the new token (K and V rows of every KV head, the index key) at position
// L = seq_len[s] and folds the index key into its block's running max (a
// fresh summary when the token opens the block).  Every chunk scores its
// blocks before own = L / B for the query at L and keeps its best K-1.  The
// scan never reads the own block's summary, so the append runs beside it.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void dstep_scan(
    const T *__restrict__ k_new, const T *__restrict__ v_new,
    const float *__restrict__ idx_k_new, T *__restrict__ k_cache,
    T *__restrict__ v_cache, float *__restrict__ idx_k_cache,
    float *__restrict__ kmax, const float *__restrict__ idx_q,
    const int64_t *__restrict__ seq_len, int64_t len_max, int64_t nb_max,
    const int32_t *__restrict__ ptab, int pt_stride, int64_t n_pages,
    int hkv, int d, int d_idx, int B, int topk, float *__restrict__ cand_s,
    int *__restrict__ cand_b, int n_chunks, int *__restrict__ run_cnt) {
  const int s = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
  const int64_t L = seq_len[s];
  // paged caches: the new token's row lives in the page of its block
  int64_t pg = 0;
  if (ptab && L >= 0 && L / B < pt_stride) pg = ptab[(int64_t)s * pt_stride + L / B];
  const bool room = L >= 0 && L < len_max && L / B < nb_max &&
                    (!ptab || (L / B < pt_stride && pg >= 0 && pg < n_pages));
  // (else: nothing is written)
  const int64_t own = room ? L / B : nb_max - 1;
  if (ch == n_chunks) {
    // the attention kernel's arrival counters of this sequence start at zero
    for (int g = tid; g < hkv; g += 256) run_cnt[(int64_t)s * hkv + g] = 0;
    if (!room) return;
    // 16-byte pieces of the K and V rows (d * sizeof(T) is a multiple of 16)
    constexpr int kV = 16 / (int)sizeof(T);
    const int vpr = d / kV;
    for (int x = tid; x < hkv * vpr; x += 256) {
      const int g = x / vpr, c = (x % vpr) * kV;
      const int64_t src = ((int64_t)s * hkv + g) * d + c;
      const int64_t dst = ptab ? ((pg * hkv + g) * B + L % B) * d + c
                               : (((int64_t)s * hkv + g) * len_max + L) * d + c;
      const uint4 kx = *reinterpret_cast<const uint4 *>(k_new + src);
      const uint4 vx = *reinterpret_cast<const uint4 *>(v_new + src);
      *reinterpret_cast<uint4 *>(k_cache + dst) = kx;
      *reinterpret_cast<uint4 *>(v_cache + dst) = vx;
    }
    float *km = kmax + ((int64_t)s * nb_max + own) * d_idx;
    const bool fresh = (L % B) == 0;
    for (int c = tid; c < d_idx; c += 256) {
      const float xv = idx_k_new[(int64_t)s * d_idx + c];
      const float old = km[c];
      if (idx_k_cache) idx_k_cache[((int64_t)s * len_max + L) * d_idx + c] = xv;
      km[c] = fresh ? xv : key2f(max(f2key(xv), f2key(old)));
    }
    return;
  }
  if (topk > 1)
    decode_scan_chunk(idx_q + (int64_t)s * d_idx, kmax + (int64_t)s * nb_max * d_idx, own,
                      nb_max, d_idx, topk - 1, ch,
                      cand_s + ((int64_t)s * n_chunks + ch) * (topk - 1),
                      cand_b + ((int64_t)s * n_chunks + ch) * (topk - 1));
}

int num_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Units of the streaming kernel: blocks are split into segments only as far
// as needed to give every other CU a unit (at most one segment per 128-key
// chunk, so the partial count stays within the workspace's topk * ceil(B/128)
// records per (sequence, query head)); at least ceil(n_seq / 6) workgroups,
// so a workgroup's units span at most kStepSeqs sequences.  Half the CUs, not
// all: at one sequence (8 blocks x 8 KV heads) two 128-key segments per block
// give 128 workgroups of two chunks and 16 partials per (sequence, KV head)
// for its last workgroup to combine, one batch of loads; four segments give
// 256 workgroups of one chunk but 32 partials, two batches (1M-token decode
// step 23.4 -> 21.4 us).
struct StreamPlan {
  int nseg, seg_len, grid;
  int64_t n_units;
  uint32_t u_q, u_r;   // units per workgroup, and the workgroups with one more
};
StreamPlan stream_plan(int32_t n_seq, int32_t hkv, int32_t B, int32_t topk) {
  StreamPlan p;
  const int nsub = (B + kSK - 1) / kSK;
  const int cus = num_cus();
  p.nseg = 1;
  while (p.nseg < nsub && (int64_t)n_seq * hkv * topk * p.nseg * 2 < cus) p.nseg *= 2;
  if (p.nseg > nsub) p.nseg = nsub;
  p.seg_len = ((nsub + p.nseg - 1) / p.nseg) * kSK;
  p.n_units = (int64_t)n_seq * hkv * topk * p.nseg;
  int64_t grid = cus;
  if (grid < (n_seq + 5) / 6) grid = (n_seq + 5) / 6;
  if (grid > p.n_units) grid = p.n_units;
  p.grid = (int)grid;
  p.u_q = (uint32_t)(p.n_units / grid);
  p.u_r = (uint32_t)(p.n_units % grid);
  return p;
}

template <typename T, int G, int D>
hipError_t launch_dec(const T *q, const T *kc, const T *vc, int32_t n_seq,
                      int64_t len_max, const int64_t *seq_len, int32_t hq,
                      int32_t hkv, int32_t B, const int32_t *sel, int32_t topk,
                      float scale, float *o, float *lse, float *part_o,
                      float *part_lse, hipStream_t st) {
  const int nsub = (B + kDK - 1) / kDK;
  int np = topk * nsub;
  if constexpr (sizeof(T) == 2 && D == 128) {
    const StreamPlan pl = stream_plan(n_seq, hkv, B, topk);
    hipLaunchKernelGGL((decode_stream<G, false>), dim3(pl.grid), dim3(256), 0, st, q, kc, vc,
                       len_max, nullptr, 0, (int64_t)0, seq_len, hq, hkv, B,
                       const_cast<int32_t *>(sel), topk, pl.nseg,
                       pl.seg_len, pl.u_q, pl.u_r, scale * kLog2e, part_o, part_lse, nullptr,
                       nullptr, 0, (int64_t)0, nullptr, nullptr, nullptr);
    hipLaunchKernelGGL((decode_merge_runs<D>), dim3(hq, n_seq), dim3(D), 0, st, G, hkv,
                       (uint32_t)(topk * pl.nseg), pl.u_q, pl.u_r, part_o, part_lse, o, lse);
    return hipGetLastError();
  } else {
    const dim3 grid(topk * nsub, hkv, n_seq);
    hipLaunchKernelGGL((decode_attn<T, G, D>), grid, dim3(256), 0, st, q, kc, vc,
                       len_max, seq_len, hq, B, sel, topk, nsub, scale * kLog2e,
                       part_o, part_lse);
  }
  hipLaunchKernelGGL((decode_merge<D>), dim3(hq, n_seq), dim3(D), 0, st,
                     np, G, hkv, part_o, part_lse, o, lse);
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

// ---------------------------------------------------------------------------
// Paged (bf16 or FP8) decode: same workspace as launch_decode.
// ---------------------------------------------------------------------------
template <int G>
void launch_paged_g(int32_t kv_dtype, const StreamPlan &pl, const uint16_t *q,
                    const uint8_t *kp, const uint8_t *vp, const float *k_scale,
                    const float *v_scale, const int32_t *block_table, int32_t max_blocks,
                    int64_t n_pages, const int64_t *seq_len, int32_t hq, int32_t hkv,
                    int32_t block, const int32_t *sel, int32_t topk, float scale,
                    float *part_o, float *part_lse, hipStream_t st) {
  if (kv_dtype == 2)
    hipLaunchKernelGGL((decode_paged_fp8<G>), dim3(pl.grid), dim3(256), 0, st, q, kp, vp,
                       k_scale, v_scale, block_table, max_blocks, n_pages, seq_len, hq, hkv,
                       block, sel, topk, pl.nseg, pl.seg_len, pl.u_q, pl.u_r, scale * kLog2e,
                       part_o, part_lse);
  else
    hipLaunchKernelGGL((decode_paged<G>), dim3(pl.grid), dim3(256), 0, st, q, kp, vp,
                       k_scale, v_scale, block_table, max_blocks, n_pages, seq_len, hq, hkv,
                       block, sel, topk, pl.nseg, pl.seg_len, pl.u_q, pl.u_r, scale * kLog2e,
                       part_o, part_lse);
}

bool decode_paged_supported(int32_t kv_dtype, int32_t d, int32_t group) {
  return (kv_dtype == 1 || kv_dtype == 2) && d == 128 &&
         (group == 1 || group == 2 || group == 4 || group == 8 || group == 16);
}

hipError_t launch_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                               int32_t kv_dtype, const float *k_scale, const float *v_scale,
                               int64_t n_pages, const int32_t *block_table, int32_t max_blocks,
                               int32_t n_seq, const int64_t *seq_len, int32_t hq, int32_t hkv,
                               int32_t block, const int32_t *sel, int32_t topk, float scale,
                               float *o, float *lse, void *ws, hipStream_t st) {
  const int G = hq / hkv;
  const int64_t np = dec_partials(n_seq, hq, block, topk);
  char *w = static_cast<char *>(ws);
  float *part_o = reinterpret_cast<float *>(w);
  w += align256((size_t)np * 128 * 4);
  float *part_lse = reinterpret_cast<float *>(w);
  const StreamPlan pl = stream_plan(n_seq, hkv, block, topk);
  const uint16_t *qq = static_cast<const uint16_t *>(q);
  const uint8_t *kp = static_cast<const uint8_t *>(k_pages);
  const uint8_t *vp = static_cast<const uint8_t *>(v_pages);
  switch (G) {
    case 1: launch_paged_g<1>(kv_dtype, pl, qq, kp, vp, k_scale, v_scale, block_table,
                              max_blocks, n_pages, seq_len, hq, hkv, block, sel, topk, scale,
                              part_o, part_lse, st); break;
    case 2: launch_paged_g<2>(kv_dtype, pl, qq, kp, vp, k_scale, v_scale, block_table,
                              max_blocks, n_pages, seq_len, hq, hkv, block, sel, topk, scale,
                              part_o, part_lse, st); break;
    case 4: launch_paged_g<4>(kv_dtype, pl, qq, kp, vp, k_scale, v_scale, block_table,
                              max_blocks, n_pages, seq_len, hq, hkv, block, sel, topk, scale,
                              part_o, part_lse, st); break;
    case 8: launch_paged_g<8>(kv_dtype, pl, qq, kp, vp, k_scale, v_scale, block_table,
                              max_blocks, n_pages, seq_len, hq, hkv, block, sel, topk, scale,
                              part_o, part_lse, st); break;
    case 16: launch_paged_g<16>(kv_dtype, pl, qq, kp, vp, k_scale, v_scale, block_table,
                                max_blocks, n_pages, seq_len, hq, hkv, block, sel, topk, scale,
                                part_o, part_lse, st); break;
    default:
      return hipErrorInvalidValue;
  }
  // one partial per run (bf16 and FP8 pages alike)
  hipLaunchKernelGGL((decode_merge_runs<128>), dim3(hq, n_seq), dim3(128), 0, st, G, hkv,
                     (uint32_t)(topk * pl.nseg), pl.u_q, pl.u_r, part_o, part_lse, o, lse);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused decode step (append, running block max, index scan, top-K, sparse
// GQA, merge) for bf16 with d = 128: two kernels, the scan (with the append)
// and the streaming attention, whose last workgroup per run merges it.
// Layout: [candidate scores][candidate ids][arrival counters][partial o]
// [partial lse].
// ---------------------------------------------------------------------------
size_t decode_step_ws_bytes(int32_t n_seq, int64_t nb_max, int32_t hq, int32_t d,
                            int32_t block, int32_t topk) {
  const int64_t n_chunks = (nb_max + kDecChunk - 1) / kDecChunk;
  const size_t nc = (size_t)n_seq * n_chunks * (topk > 1 ? topk - 1 : 1);
  // + one arrival counter per (sequence, KV head); Hq bounds Hkv
  return align256(nc * 4) + align256(nc * 4) + align256((size_t)n_seq * hq * 4) +
         decode_ws_bytes(n_seq, hq, d, block, topk);
}

bool decode_step_supported(int32_t dtype, int32_t d, int32_t group) {
  return dtype == 1 && d == 128 &&
         (group == 1 || group == 2 || group == 4 || group == 8 || group == 16);
}

hipError_t launch_decode_step(const void *q, const void *k_new, const void *v_new,
                              const float *idx_q, const float *idx_k_new, void *k_cache,
                              void *v_cache, const int32_t *ptab, int32_t pt_stride,
                              int64_t n_pages, float *idx_k_cache, float *kmax,
                              int32_t n_seq, int64_t len_max, int64_t nb_max,
                              const int64_t *seq_len, int32_t hq, int32_t hkv, int32_t d,
                              int32_t d_idx, int32_t block, int32_t topk, float scale,
                              int32_t *sel, float *o, float *lse, void *ws,
                              hipStream_t st) {
  const int G = hq / hkv;
  const int n_chunks = (int)((nb_max + kDecChunk - 1) / kDecChunk);
  const size_t nc = (size_t)n_seq * n_chunks * (topk > 1 ? topk - 1 : 1);
  char *w = static_cast<char *>(ws);
  float *cand_s = reinterpret_cast<float *>(w);
  w += align256(nc * 4);
  int *cand_b = reinterpret_cast<int *>(w);
  w += align256(nc * 4);
  int *run_cnt = reinterpret_cast<int *>(w);
  w += align256((size_t)n_seq * hq * 4);
  const int64_t np_max = dec_partials(n_seq, hq, block, topk);
  float *part_o = reinterpret_cast<float *>(w);
  w += align256((size_t)np_max * d * 4);
  float *part_lse = reinterpret_cast<float *>(w);

  const uint16_t *qq = static_cast<const uint16_t *>(q);
  uint16_t *kc = static_cast<uint16_t *>(k_cache);
  uint16_t *vc = static_cast<uint16_t *>(v_cache);
  hipLaunchKernelGGL((dstep_scan<uint16_t>), dim3(n_chunks + 1, n_seq), dim3(256), 0, st,
                     static_cast<const uint16_t *>(k_new), static_cast<const uint16_t *>(v_new),
                     idx_k_new, kc, vc, idx_k_cache, kmax, idx_q, seq_len, len_max, nb_max,
                     ptab, pt_stride, n_pages, hkv, d, d_idx, block, topk, cand_s, cand_b,
                     n_chunks, run_cnt);
  const StreamPlan pl = stream_plan(n_seq, hkv, block, topk);
#define MSA_STEP_CASE(GG)                                                               \
  case GG:                                                                              \
    hipLaunchKernelGGL((decode_stream<GG, true>), dim3(pl.grid), dim3(256), 0, st, qq, kc, \
                       vc, len_max, ptab, pt_stride, n_pages, seq_len, hq, hkv, block, sel, \
                       topk, pl.nseg,                                                    \
                       pl.seg_len, pl.u_q, pl.u_r, scale * kLog2e, part_o, part_lse, cand_s, \
                       cand_b, n_chunks, nb_max, run_cnt, o, lse);                       \
    break;
  switch (G) {
    MSA_STEP_CASE(1)
    MSA_STEP_CASE(2)
    MSA_STEP_CASE(4)
    MSA_STEP_CASE(8)
    MSA_STEP_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef MSA_STEP_CASE
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of msa_decode_step_noalloc: a file-scope device array (each device
// the library runs on holds its own copy until the process ends).  Its device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and kept; kernels get that address, never the array's name
// (which in host code is only a stand-in).  The decode step writes every
// scratch word it reads before reading it, so nothing needs clearing; calls
// that overlap on one device share the array and race.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t noalloc_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {nullptr};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace msa

