// prefill_mfma.hip -- sparse-branch prefill on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16), d = 128.  Same two-pass KV-outer organisation
// as the VALU kernels in prefill.hip (sparse branch of "MiniMax M3模型算力成本
// 大幅降低原因深度解析"; section 2.2 "KV Outer Gather Q：MSA 的关键设计" of
// chenxutan.com's "MiniMax M3 深度实战"):
//   pass A  work items (KV block b, KV head g, tile of 256/G queries from
//           row b's non-own list), walked by a persistent grid of 8-wave
//           workgroups: K[g,b] and V[g,b] are streamed into LDS in 128-key
//           chunks and applied to all 256 gathered query rows (tile tokens x
//           the G query heads of group g);
//   pass B  one 4-wave workgroup per (block b, head g, tile of b's own
//           tokens): causal attention inside the own block (64-key chunks),
//           then the log-sum-exp merge with pass A's partials; writes O and
//           LSE.
//
// Each wave owns NB = 1 32-row N-block, and each SIMD runs two waves, so one
// wave's softmax overlaps the other's MFMAs.  Scores are computed transposed, S^T = K Q^T
// (keys = MFMA rows), so a lane holds 16 keys of ONE query row: the row max
// needs one v_permlane32_swap with lane l^32 and the softmax statistics stay
// per lane.  P^T leaves the accumulator already in the B-operand layout of
// O^T = V^T P^T, provided V^T's k-slots follow the same key order: V is
// staged row-major in LDS and each V^T operand is read with two
// ds_read_b64_tr_b16 (each 16-lane group reads a 4-key x 16-column tile
// transposed, so lane i gets column i of four consecutive keys).  Lazy
// rescaling keeps every weight at most 2^8 and removes most O rescales: in
// pass B the running reference max moves only when a row's max exceeds it by
// more than 8; in pass A the weights are first taken against the reference
// and the row max is only computed when a lane's 16 weights sum past 2^8.
#include <type_traits>

#include "msa_internal.h"
#include "prefill_common.h"
#include "mfma_common.h"
#include "seqtab.h"

namespace msa {
namespace {

constexpr int kD = 128;          // head dim handled here
constexpr int kKC = 64;          // keys per staged chunk
constexpr int kKStr = kD + 8;    // K row stride in LDS, bf16 elements (272 B)
constexpr int kVStr = kD + 16;   // V row stride in LDS, bf16 elements (288 B)
constexpr float kLazy = 8.f;     // reference-max slack (log2 units)

struct MfmaSmem {
  uint16_t Ks[kKC * kKStr];
  uint16_t Vs[kKC * kVStr];
};

// Staging of one 64-key chunk of a (head, block) slice, split so the global
// loads of chunk i+1 are in flight while chunk i is computed: load() fills
// registers, store() writes K and V row-major (padded rows) into one of the
// two LDS buffers.  Rows past nrows are zero.
template <int NT>
struct ChunkRegs {
  static constexpr int kIt = (kKC * kD / 8) / NT;   // 16-byte pieces per thread
  u32x4 k[kIt], v[kIt];
};

template <int NT>
__device__ __forceinline__ void load_chunk(ChunkRegs<NT> &cr, const uint16_t *k,
                                           const uint16_t *v, int64_t row0,
                                           int nrows) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < ChunkRegs<NT>::kIt; ++it) {
    const int x = tid + NT * it;
    const int key = x >> 4, seg = x & 15;
    u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (key < nrows) {
      kv = *reinterpret_cast<const u32x4 *>(k + (row0 + key) * kD + seg * 8);
      vv = *reinterpret_cast<const u32x4 *>(v + (row0 + key) * kD + seg * 8);
    }
    cr.k[it] = kv;
    cr.v[it] = vv;
  }
}

template <int NT>
__device__ __forceinline__ void store_chunk(MfmaSmem &sm, const ChunkRegs<NT> &cr) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < ChunkRegs<NT>::kIt; ++it) {
    const int x = tid + NT * it;
    const int key = x >> 4, seg = x & 15;
    *reinterpret_cast<u32x4 *>(&sm.Ks[key * kKStr + seg * 8]) = cr.k[it];
    *reinterpret_cast<u32x4 *>(&sm.Vs[key * kVStr + seg * 8]) = cr.v[it];
  }
}

// Offset of element (pair n, head g*G+hl, column c = cb*32 + 8*rg + 4*hf + e)
// in the partial-output workspace.  The order follows the O^T accumulator
// fragments, so that the 2*G lanes holding one token's rows in a wave read or
// write 32*G contiguous bytes per (cb, rg): [n][g][cb][rg][hf][hl][e].
__device__ __forceinline__ int64_t frag_off(int64_t n, int g, int hq, int G,
                                            int hl, int cb, int rg, int hf) {
  return n * (int64_t)hq * kD + (int64_t)g * G * kD + cb * 32 * G + rg * 8 * G +
         hf * 4 * G + hl * 4;
}

// A partial record of one (pair, query head): the normalised output o as
// fp16 scaled by 2^-e, where 2^e is the smallest power of two above max|o|
// (so every stored value is below 1 in magnitude -- no overflow -- and the
// relative precision is 2^-11 of max|o|), plus (lse, e) as a float2.  The
// merge weight of the record is 2^(lse - M) for the normaliser and
// 2^(lse + e - M) for the stored values.
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void put_partial(uint16_t *part_o, float2 *part_le,
                                            int64_t n, int g, int hq, int G,
                                            int hl, int hf, const f32x16 (&acc)[4],
                                            float mref, float ltot) {
  const float inv = 1.f / ltot;
  float mabs = 0.f;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mabs = fmaxf(mabs, fabsf(acc[cb][r]));
  mabs = max_with_partner(mabs * inv);
  int e = 0;
  if (mabs > 0.f) (void)frexpf(mabs, &e);
  const float f = ldexpf(inv, -e);
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      float4 v = make_float4(acc[cb][4 * rg] * f, acc[cb][4 * rg + 1] * f,
                             acc[cb][4 * rg + 2] * f, acc[cb][4 * rg + 3] * f);
      const f16x4 hv = {(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
      *reinterpret_cast<f16x4 *>(part_o + frag_off(n, g, hq, G, hl, cb, rg, hf)) = hv;
    }
  if (hf == 0) part_le[n * hq + (int64_t)g * G + hl] = make_float2(mref + __log2f(ltot), (float)e);
}

// Own-block pass: workgroup = (tile of TPT own tokens of one query-holding
// block of one sequence, KV head g).  NB = 32-row N-blocks per wave, NW =
// waves per workgroup.  At most 256 registers per lane (two waves per SIMD):
// with NW = 4, two workgroups share a CU, so one's merge loads overlap the
// other's matrix-core work.  Query rows, selections, slots, outputs and CSR
// positions are those of the whole chain (global); blocks in sel are local
// to the query's sequence.
template <int G, int NB, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void prefill_mfma_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, KvMap kvm, SeqTab tab, int hq,
    const int32_t *__restrict__ sel, int topk, const int32_t *__restrict__ slot,
    float scale_log2, uint16_t *__restrict__ part_o, float2 *__restrict__ part_le,
    int64_t n_part, float *__restrict__ o, float *__restrict__ lse) {
  constexpr int NT = 64 * NW;    // threads
  constexpr int TPN = 32 / G;    // tokens per 32-row N-block
  constexpr int TPW = NB * TPN;  // tokens per wave
  constexpr int TPT = NW * TPW;  // tokens per tile (workgroup)
  __shared__ MfmaSmem smb[2];

  // XCD-aware order: workgroups are dealt to the eight XCDs round-robin by
  // linear id, so linear id L runs work item L' = the (L / 8)-th of the L % 8-th
  // eighth of all (tile, KV head) items.  Each XCD then walks a contiguous
  // range -- every tile of a block and head on one XCD, whose L2 holds that
  // block's keys and values for all of them.
  const uint64_t n_items = (uint64_t)gridDim.x * gridDim.y;
  const uint64_t lin = blockIdx.x + (uint64_t)blockIdx.y * gridDim.x;
  const uint64_t xq = n_items / 8, xr = n_items % 8, xc = lin % 8, xk = lin / 8;
  const uint64_t item = (xc < xr ? xc * (xq + 1) : xr * (xq + 1) + (xc - xr) * xq) + xk;
  const int64_t tile_x = (int64_t)(item % gridDim.x);
  const int g = (int)(item / gridDim.x);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = lane >> 5, j = lane & 31;

  // ---- the tile: sequence s, its block b, the key count, each row's query ----
  const int B = tab.B;
  const int tpb = (B + TPT - 1) / TPT;
  const int64_t bt = tile_x / tpb;   // query-holding block of the chain
  const int sq = prefix_find(tab.ob0, tab.n, bt);
  const int64_t q_pos0 = tab.q_pos0[sq], n_q = seq_nq(tab, sq), row0 = tab.q_row0[sq];
  const int64_t b = q_pos0 / B + (bt - tab.ob0[sq]);
  const int64_t tok0 = b * B + (int64_t)(tile_x % tpb) * TPT;
  int64_t hi = tok0 + TPT - 1;
  if (hi > b * B + B - 1) hi = b * B + B - 1;
  if (hi > q_pos0 + n_q - 1) hi = q_pos0 + n_q - 1;
  if (hi < tok0 || hi < q_pos0) return;
  const int64_t nkeys = hi - b * B + 1;
  const int64_t min_pos = tok0;

  int64_t qi[NB], pos[NB];
  bool act[NB];
  int head[NB];
  bf16x8 qf[NB][8];
#pragma unroll
  for (int nbk = 0; nbk < NB; ++nbk) {
    const int tl = wave * TPW + nbk * TPN + j / G;
    head[nbk] = j % G;
    const int64_t p = tok0 + tl;
    act[nbk] = p >= q_pos0 && p < q_pos0 + n_q && p < b * B + B;
    pos[nbk] = p < b * B + B ? p : b * B + B - 1;
    qi[nbk] = act[nbk] ? row0 + (p - q_pos0) : 0;   // query row of the chain
    const uint16_t *qp = q + ((qi[nbk] * hq + (int64_t)g * G + head[nbk]) * kD);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (act[nbk]) x = *reinterpret_cast<const u32x4 *>(qp + cc * 16 + 8 * h);
      qf[nbk][cc] = as_bf16x8(x);
    }
  }

  f32x16 acc[NB][4];
#pragma unroll
  for (int nbk = 0; nbk < NB; ++nbk)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nbk][cb][r] = 0.f;
  float mref[NB], lsum[NB];
#pragma unroll
  for (int nbk = 0; nbk < NB; ++nbk) {
    mref[nbk] = -INFINITY;
    lsum[nbk] = 0.f;
  }

  // the own block's keys and values (rows 0 .. nkeys-1 from these)
  const int64_t kvo = kv_block_off<kD>(kvm, tab, sq, b, g);
  const uint16_t *kb = k + kvo;
  const uint16_t *vb = v + kvo;
  const int64_t n_chunks = (nkeys + kKC - 1) / kKC;
  ChunkRegs<NT> cr;
  load_chunk(cr, kb, vb, 0, (int)(nkeys < kKC ? nkeys : kKC));
  store_chunk(smb[0], cr);
  __syncthreads();
  for (int64_t ci = 0; ci < n_chunks; ++ci) {
    const int64_t kc = ci * kKC;
    if (ci + 1 < n_chunks) {
      const int64_t nxt = kc + kKC;
      load_chunk(cr, kb, vb, nxt,
                 (int)(nkeys - nxt < kKC ? nkeys - nxt : kKC));
    }
    MfmaSmem &sm = smb[ci & 1];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int koff0 = (int)kc + sub * 32;          // key offset in block
      if (koff0 >= nkeys) break;
      f32x16 s[NB];
#pragma unroll
      for (int nbk = 0; nbk < NB; ++nbk)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nbk][r] = 0.f;
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const u32x4 kraw = *reinterpret_cast<const u32x4 *>(
            &sm.Ks[(sub * 32 + j) * kKStr + cc * 16 + 8 * h]);
        const bf16x8 kf = as_bf16x8(kraw);
#pragma unroll
        for (int nbk = 0; nbk < NB; ++nbk) s[nbk] = mfma32(kf, qf[nbk][cc], s[nbk]);
      }
      const bool need_mask = koff0 + 31 >= nkeys || b * B + koff0 + 31 > min_pos;
      bf16x8 pb[NB][2];
#pragma unroll
      for (int nbk = 0; nbk < NB; ++nbk) {
        if (need_mask) {
          const int64_t lim = pos[nbk] - b * B;
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
        mloc = max_with_partner(mloc);
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
      // V^T operand rows: this lane's 16-lane group reads keys
      // sub*32 + 16ks + 4h + a/4 (+8), columns cb*32 + 16*(j/16) + 4*(a%4)
      const int a16 = lane & 15;
      const uint16_t *vbase = &sm.Vs[(sub * 32 + 4 * h + (a16 >> 2)) * kVStr +
                                     16 * (j >> 4) + 4 * (a16 & 3)];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const uint16_t *vr = vbase + 16 * ks * kVStr + cb * 32;
          const u32x2 lo = lds_read_tr(vr);
          const u32x2 hi = lds_read_tr(vr + 8 * kVStr);
          const u32x4 vraw = {lo[0], lo[1], hi[0], hi[1]};
          const bf16x8 vf = as_bf16x8(vraw);
#pragma unroll
          for (int nbk = 0; nbk < NB; ++nbk)
            acc[nbk][cb] = mfma32(vf, pb[nbk][ks], acc[nbk][cb]);
        }
      }
    }
    if (ci + 1 < n_chunks) store_chunk(smb[(ci + 1) & 1], cr);
    __syncthreads();
  }

  // ---- epilogue ----
#pragma unroll
  for (int nbk = 0; nbk < NB; ++nbk) {
    const float ltot = sum_with_partner(lsum[nbk]);
    const int hh = g * G + head[nbk];
    {
      if (!act[nbk]) continue;
      const int64_t i = qi[nbk];
      const int32_t *srow = sel + i * topk;
      const int32_t *xrow = slot + i * topk;
      const float own2 = mref[nbk] + __log2f(ltot);
      float z, mx = own2;
      if (topk <= 16) {
        // the query's non-own records, every load of a stage issued together
        // (K <= 16): the record indices, then all (lse, e) pairs, then the fp16
        // outputs two records at a time; larger K merges record by record
        constexpr int kMaxM = 16;
        int64_t nid[kMaxM];
#pragma unroll
        for (int kk = 0; kk < kMaxM; ++kk) {
          nid[kk] = -1;
          if (kk < topk) {
            const int32_t bk = srow[kk], x = xrow[kk];
            if (bk >= 0 && bk < b) {
              const int64_t n = x - own_through_g(tab, sq, bk);
              if (n >= 0 && n < n_part) nid[kk] = n;
            }
          }
        }
        float2 le[kMaxM];
#pragma unroll
        for (int kk = 0; kk < kMaxM; ++kk)
          le[kk] = nid[kk] >= 0 ? part_le[nid[kk] * hq + hh] : make_float2(-INFINITY, 0.f);
#pragma unroll
        for (int kk = 0; kk < kMaxM; ++kk) mx = fmaxf(mx, le[kk].x);
        z = fast_exp2(own2 - mx);
        const float wo = z / ltot;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[nbk][cb][r] *= wo;
#pragma unroll
        for (int k0 = 0; k0 < kMaxM; k0 += 2) {
          if (k0 >= topk) break;
          f16x4 pv[2][16];
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int f = 0; f < 16; ++f) {
              pv[u][f] = f16x4{0, 0, 0, 0};
              if (nid[k0 + u] >= 0)
                pv[u][f] = *reinterpret_cast<const f16x4 *>(
                    part_o + frag_off(nid[k0 + u], g, hq, G, head[nbk], f >> 2, f & 3, h));
            }
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            if (nid[k0 + u] < 0) continue;
            z += fast_exp2(le[k0 + u].x - mx);
            const float wk = fast_exp2(le[k0 + u].x + le[k0 + u].y - mx);
#pragma unroll
            for (int f = 0; f < 16; ++f) {
              const int cb = f >> 2, rg = f & 3;
              acc[nbk][cb][4 * rg] = fmaf(wk, (float)pv[u][f].x, acc[nbk][cb][4 * rg]);
              acc[nbk][cb][4 * rg + 1] = fmaf(wk, (float)pv[u][f].y, acc[nbk][cb][4 * rg + 1]);
              acc[nbk][cb][4 * rg + 2] = fmaf(wk, (float)pv[u][f].z, acc[nbk][cb][4 * rg + 2]);
              acc[nbk][cb][4 * rg + 3] = fmaf(wk, (float)pv[u][f].w, acc[nbk][cb][4 * rg + 3]);
            }
          }
        }
      } else {
        for (int kk = 0; kk < topk; ++kk) {
          const int32_t bk = srow[kk];
          if (bk < 0 || bk >= b) continue;
          const int64_t n_idx = xrow[kk] - own_through_g(tab, sq, bk);
          if (n_idx < 0 || n_idx >= n_part) continue;
          mx = fmaxf(mx, part_le[n_idx * hq + hh].x);
        }
        z = fast_exp2(own2 - mx);
        const float wo = z / ltot;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[nbk][cb][r] *= wo;
        for (int kk = 0; kk < topk; ++kk) {
          const int32_t bk = srow[kk];
          if (bk < 0 || bk >= b) continue;
          const int64_t n_idx = xrow[kk] - own_through_g(tab, sq, bk);
          if (n_idx < 0 || n_idx >= n_part) continue;
          const float2 le = part_le[n_idx * hq + hh];
          z += fast_exp2(le.x - mx);
          const float wk = fast_exp2(le.x + le.y - mx);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
              const f16x4 pv = *reinterpret_cast<const f16x4 *>(
                  part_o + frag_off(n_idx, g, hq, G, head[nbk], cb, rg, h));
              acc[nbk][cb][4 * rg] = fmaf(wk, (float)pv.x, acc[nbk][cb][4 * rg]);
              acc[nbk][cb][4 * rg + 1] = fmaf(wk, (float)pv.y, acc[nbk][cb][4 * rg + 1]);
              acc[nbk][cb][4 * rg + 2] = fmaf(wk, (float)pv.z, acc[nbk][cb][4 * rg + 2]);
              acc[nbk][cb][4 * rg + 3] = fmaf(wk, (float)pv.w, acc[nbk][cb][4 * rg + 3]);
            }
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

// ---------------------------------------------------------------------------
// Asynchronous chunk staging for the persistent pass: a buffer load with the
// LDS bit copies 16 bytes per lane straight into LDS at base + 16 * lane, so one wave
// instruction fills four 256-byte rows; each lane picks which global segment
// lands in its slot.  Rows are unpadded and XOR-swizzled by segment instead:
//   K: segment s of row r at slot s ^ (r & 15)  -- the 16 rows read by a
//      16-lane group for an A operand hit 16 distinct bank groups;
//   V: segment s of row r at slot s ^ 4(r & 3) -- a half-wave of a
//      ds_read_b64_tr_b16 reads 4 consecutive rows x 4 segments (one aligned
//      group of four), and the XOR moves each row to its own group of four
//      slots, so the 32 lanes cover all 64 banks once; rows 4 apart share the
//      pattern, so all of a lane's V reads sit at constant offsets from one
//      address per column block.
// Rows past a short chunk are out of the buffer's range and fetch nothing;
// their LDS rows hold zeros (the buffers start zeroed) or an earlier chunk's
// rows -- finite either way, so the masked keys' zero weights add nothing.
// Chunks are kKA = 128 keys (64 KiB of K and V), two in LDS: one computed
// while the next streams in.
// ---------------------------------------------------------------------------
constexpr int kKA = 128;   // keys per staged chunk, persistent pass
constexpr float kCap = 256.f;   // bound on a lane's weight sum per sub-tile

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Sum of the 16 bf16 weights of a lane (the values the P*V product uses),
// in fp32 on v_dot2 against ones.
__device__ __forceinline__ float row_sum16(bf16x8 a, bf16x8 b) {
  const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[2 * i], a[2 * i + 1]}, one, s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{b[2 * i], b[2 * i + 1]}, one, s1, false);
  }
  return s0 + s1;
}

struct AsyncSmem {
  uint16_t Ks[kKA * kD];
  uint16_t Vs[kKA * kD];
};

typedef __attribute__((address_space(1))) void *gptr_t;
typedef __attribute__((address_space(3))) void *lptr_t;

__device__ __forceinline__ int kswz(int r, int sgm) { return sgm ^ (r & 15); }
__device__ __forceinline__ int vswz(int r, int sgm) { return sgm ^ (4 * (r & 3)); }

// Each 16-byte piece of a chunk goes by a buffer load straight into LDS: the
// chunk's first row is the buffer base (scalar registers) and its nrows rows
// the buffer's range, so a lane's source offset depends on its slot only.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const uint16_t *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(p), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, lptr_t dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
}

// One chunk (nrows <= kKA keys of K and of V) into LDS: every lane copies
// 16-byte pieces, (kKA * kD / 8) / (64 * NW) of K and as many of V.  Piece
// (row r, segment sp) lands at the row's swizzled slot.  Rows past nrows
// (a short block) lie beyond the buffer resource's range of nrows rows, so
// their copies fetch nothing from memory (an out-of-range buffer read yields
// zero); those keys are masked.  The offsets are
// recomputed per copy (a few integer operations) rather than kept in
// registers across the chunk loop.
template <int NW>
__device__ __forceinline__ void async_chunk(AsyncSmem &sm, const uint16_t *k,
                                            const uint16_t *v, int64_t row0, int nrows) {
  constexpr int IPW = (kKA * kD / 8) / (64 * NW);   // copies per lane, per operand
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t bytes = (uint32_t)nrows * kD * 2;
  const __amdgpu_buffer_rsrc_t rk = chunk_rsrc(k + row0 * kD, bytes);
  const __amdgpu_buffer_rsrc_t rv = chunk_rsrc(v + row0 * kD, bytes);
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int inst = wave * IPW + i;
    const int r = (inst * 64 + lane) >> 4, sp = lane & 15;
    lds_dma16(rk, (lptr_t)(&sm.Ks[inst * 64 * 8]), (uint32_t)(r * kD + kswz(r, sp) * 8) * 2);
    lds_dma16(rv, (lptr_t)(&sm.Vs[inst * 64 * 8]), (uint32_t)(r * kD + vswz(r, sp) * 8) * 2);
  }
}

// Wait for this thread's outstanding loads (the async copies included), then
// publish the LDS tile to the workgroup.
__device__ __forceinline__ void async_wait_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Pass A, persistent.  One workgroup per CU walks a static range of work
// items w = (KV head g, tile t); the range of workgroup i is the i%8-th
// eighth of all items, so the workgroups placed on one XCD share its L2 over
// a window of consecutive tiles (same head, mostly the same KV block).  The
// next item's metadata, query fragments and first K/V chunk are fetched while
// the current item computes.
//
// Per-tile metadata (built by prefill_tile_info): info[t] = (global block,
// first CSR position, row end, sequence) and tq[t][i] = query row of the
// tile's i-th row token (-1 past the row end).
// ---------------------------------------------------------------------------
// Per-tile metadata of the KV-outer pass, everything an item needs resolved
// here once per tile, so the persistent kernel's prefetch of the next items
// is a few independent loads: the element offset of the tile's block in KV
// head 0 (head g adds g times the head stride), the partial-record index of
// the tile's first row (record of row i = nb0 + i), and the block's key count.
struct __attribute__((aligned(16))) TileMeta {
  int64_t kvb;
  int64_t nb0;
  int32_t nkeys;
  int32_t pad[3];
};

template <int TPT>
__global__ __launch_bounds__(256) void prefill_tile_info(
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ tile_ptr,
    const int32_t *__restrict__ q_list, SeqTab tab, KvMap kvm, TileMeta *__restrict__ info,
    int32_t *__restrict__ tq) {
  const int64_t gb = blockIdx.x;
  const int32_t t0 = tile_ptr[gb], t1 = tile_ptr[gb + 1];
  if (t0 == t1) return;
  const int sq = prefix_find(tab.blk0, tab.n, gb);
  const int64_t b = gb - tab.blk0[sq];
  const int64_t own_b = own_through_g(tab, sq, b) - own_through_g(tab, sq, b - 1);
  const int32_t base = (int32_t)(row_ptr[gb] + own_b), end = row_ptr[gb + 1];
  int64_t nkeys = tab.B;   // a non-own block is always full
  if (!kvm.pages) {        // contiguous rows: never past the cache (invalid input only)
    const int64_t r0 = tab.kv_row0[sq] + b * tab.B;
    if (r0 + nkeys > kvm.kv_stride) nkeys = kvm.kv_stride - r0;
    if (nkeys < 0) nkeys = 0;
  }
  const int64_t kvb = kv_block_off<kD>(kvm, tab, sq, b, 0);
  const int64_t own_thr = own_through_g(tab, sq, b);
  for (int x = threadIdx.x; x < (t1 - t0) * TPT; x += 256) {
    const int tt = x / TPT, i = x % TPT;
    const int32_t e = base + tt * TPT + i;
    tq[(int64_t)(t0 + tt) * TPT + i] = e < end ? q_list[e] : -1;
    if (i == 0) {
      TileMeta m;
      m.kvb = kvb;
      m.nb0 = (int64_t)(base + tt * TPT) - own_thr;
      m.nkeys = (int32_t)nkeys;
      m.pad[0] = m.pad[1] = m.pad[2] = 0;
      info[t0 + tt] = m;
    }
  }
}

template <int G, int NW>
__global__ __launch_bounds__(64 * NW) void prefill_nonown_persistent(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, KvMap kvm, SeqTab tab, int hq, int hkv,
    const int32_t *__restrict__ tile_ptr, const TileMeta *__restrict__ info,
    const int32_t *__restrict__ tq,
    float scale_log2, uint16_t *__restrict__ part_o, float2 *__restrict__ part_le,
    int64_t n_part) {
  constexpr int TPN = 32 / G;
  constexpr int TPT = NW * TPN;
  // Two distinct LDS buffers, each chunk step naming its own at compile
  // time: the compiler can then tell that the DMA filling one buffer does not
  // alias the transposed reads of the other, and adds no wait for it.
  __shared__ AsyncSmem sm0;
  __shared__ AsyncSmem sm1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = lane >> 5, j = lane & 31;
  const int tl = wave * TPN + j / G;  // token slot of this lane's row
  const int hl = j % G;                // head of this lane's row in the group

  // A short block's rows past its keys read as out of range: their LDS rows
  // then hold zeros or what an earlier chunk left there -- finite either
  // way, so the masked keys' zero weights times those values add nothing.
  for (int x = threadIdx.x; x < kKA * kD / 8; x += 64 * NW) {
    reinterpret_cast<u32x4 *>(sm0.Ks)[x] = u32x4{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4 *>(sm0.Vs)[x] = u32x4{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4 *>(sm1.Ks)[x] = u32x4{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4 *>(sm1.Vs)[x] = u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  const int B = tab.B;
  const int64_t n_q = tab.q_row0[tab.n];   // query rows of the chain
  const int64_t T = tile_ptr[tab.blk0[tab.n]];
  const int64_t W = T * hkv;
  const int xcd = blockIdx.x & 7;
  const int64_t per = gridDim.x >> 3, r = blockIdx.x >> 3;
  const int64_t w_end = W * (xcd + 1) / 8;
  int64_t w = W * xcd / 8 + r;
  if (w >= w_end) return;

  // Query fragments of the next item: plain loads into registers, issued at
  // the start of the current item's last chunk and first used after that
  // chunk's barrier (whose wait covers them).
  u32x4 qn[8];
  auto stage_q = [&](int gg, int32_t qr) {
    const bool a = qr >= 0 && qr < n_q;
    const uint16_t *qp = q + (((a ? (int64_t)qr : 0) * hq + (int64_t)gg * G + hl) * kD);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) qn[cc] = *reinterpret_cast<const u32x4 *>(qp + cc * 16 + 8 * h);
  };
  // A row past the tile's queries keeps the fragments of query row 0 (a
  // valid row, so its scores are finite); its results are never stored.
  auto read_q = [&](int32_t qr, bf16x8 (&dst)[8]) {
    (void)qr;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) dst[cc] = as_bf16x8(qn[cc]);
  };
  // element offset of an item's block in KV head gg, and its key count
  const int64_t hstride = kvm.pages ? (int64_t)B * kD : kvm.kv_stride * kD;
  auto kv_off = [&](const TileMeta &f, int gg) { return f.kvb + (int64_t)gg * hstride; };
  auto kv_keys = [&](const TileMeta &f) { return (int64_t)f.nkeys; };

  // current item: head, tile info, this lane's query, K/V span
  int g = (int)(w / T);
  TileMeta inf = info[w % T];
  int32_t qraw = tq[(w % T) * TPT + tl];
  int64_t nkeys = kv_keys(inf);
  int64_t n_chunks = (nkeys + kKA - 1) / kKA;
  int64_t ci = 0;
  stage_q(g, qraw);
  int64_t kvo = kv_off(inf, g);
  async_chunk<NW>(sm0, k + kvo, v + kvo, 0, (int)(nkeys < kKA ? nkeys : kKA));
  // Metadata of the next item.  The one after it is fetched at the start of
  // each item's last chunk, so the load completes under that chunk's
  // compute and is only moved into place after the chunk's barrier.
  int64_t wn = w + per;
  bool has_next = wn < w_end;
  int gn = 0;
  TileMeta infn = {};
  int32_t qrawn = -1;
  auto fetch = [&](int64_t ww, int &gg, TileMeta &ii, int32_t &qq) {
    if (ww < w_end) {
      gg = (int)(ww / T);
      ii = info[ww % T];
      qq = tq[(ww % T) * TPT + tl];
    }
  };
  fetch(wn, gn, infn, qrawn);
  async_wait_barrier();

  // Byte offsets of this lane's V^T pieces in a chunk, per column block cb:
  // its 16-lane group reads 4 keys x 16 columns; lane a16 supplies key
  // (a16 / 4) and the 8-byte piece a16 % 4.  The second piece of a k-step is
  // 8 keys further, the next k-step 16, the next sub-tile 32 (constant
  // offsets: the swizzle repeats every 4 rows).  Keeping each read one
  // constant away from the buffer base keeps the compiler's alias
  // information for it.
  int voff[4];
  {
    const int a16 = lane & 15;
    const int vrow = 4 * h + (a16 >> 2);
    const int vcol0 = 16 * (j >> 4) + 4 * (a16 & 3);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int col = cb * 32 + vcol0;
      voff[cb] = (vrow * kD + vswz(vrow, col >> 3) * 8 + (col & 7)) * 2;
    }
  }

  bf16x8 qf[8];
  read_q(qraw, qf);
  f32x16 acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) acc[cb][rr] = 0.f;
  float mref = -INFINITY, lsum = 0.f;

  // One chunk of the current item on buffer P, with the next chunk
  // (or the next item's first chunk and queries) streaming into the other.
  // Returns false once this workgroup's range is done.
  auto step = [&](auto tag) -> bool {
    constexpr int P = decltype(tag)::value;
    AsyncSmem &cur = P ? sm1 : sm0;
    AsyncSmem &nxt = P ? sm0 : sm1;
    const int64_t kc = ci * kKA;
    const bool last = ci + 1 >= n_chunks;
    int gnn = 0;
    TileMeta infnn = {};
    int32_t qrawnn = -1;
    if (last && has_next) {
      stage_q(gn, qrawn);
      fetch(wn + per, gnn, infnn, qrawnn);
    }
    if (!last) {
      const int64_t nxt_row = kc + kKA;
      async_chunk<NW>(nxt, k + kvo, v + kvo, nxt_row,
                      (int)(nkeys - nxt_row < kKA ? nkeys - nxt_row : kKA));
    } else if (has_next) {
      const int64_t nk = kv_keys(infn);
      const int64_t kvn = kv_off(infn, gn);
      async_chunk<NW>(nxt, k + kvn, v + kvn, 0, (int)(nk < kKA ? nk : kKA));
    }
#pragma unroll
    for (int sub = 0; sub < kKA / 32; ++sub) {
      const int koff0 = (int)kc + sub * 32;
      if (koff0 >= nkeys) break;
      f32x16 sacc;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sacc[rr] = 0.f;
      // all eight K operands of the sub-tile are read before its first
      // product, so the LDS round trips overlap instead of stalling each
      // product of the dependent Q.K^T chain
      u32x4 kpre[8];
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const int kr = sub * 32 + j;
        kpre[cc] = *reinterpret_cast<const u32x4 *>(
            &cur.Ks[kr * kD + kswz(kr, cc * 2 + h) * 8]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) sacc = mfma32(as_bf16x8(kpre[cc]), qf[cc], sacc);
      if (koff0 + 31 >= nkeys) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int koff = koff0 + 8 * (rr >> 2) + 4 * h + (rr & 3);
          if (koff >= nkeys) sacc[rr] = -INFINITY;
        }
      }
      // Weights against the current reference max; after an item's first
      // sub-tile (which takes its row max as the reference) the row max is
      // only computed when some lane's 16 weights sum past 2^8, which bounds
      // every weight by 2^8 as a per-sub-tile max test would.
      bf16x8 pb0, pb1;
      float ps;
      auto weights = [&]() {
        f32x8 p0, p1;
        const float nm = -mref;
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          p0[rr] = fast_exp2(fmaf(sacc[rr], scale_log2, nm));
          p1[rr] = fast_exp2(fmaf(sacc[rr + 8], scale_log2, nm));
        }
        pb0 = __builtin_convertvector(p0, bf16x8);
        pb1 = __builtin_convertvector(p1, bf16x8);
        ps = row_sum16(pb0, pb1);
      };
      // V^T operands of the first k-step, read ahead of the softmax: their
      // LDS round trip runs under its exponentials
      const char *vbase = reinterpret_cast<const char *>(cur.Vs);
      u32x4 vpre[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        constexpr int kRow = kD * 2;
        const int o0 = voff[cb] + (sub * 32) * kRow;
        const u32x2 lo = lds_read_tr(reinterpret_cast<const uint16_t *>(vbase + o0));
        const u32x2 hi = lds_read_tr(reinterpret_cast<const uint16_t *>(vbase + o0 + 8 * kRow));
        vpre[cb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
      __builtin_amdgcn_sched_barrier(0);
      if (sub == 0 && ci == 0) {
        // an item's first sub-tile: the reference max is its own row max, so
        // its weights are taken once (the test below then passes)
        float m0 = sacc[0];
#pragma unroll
        for (int rr = 1; rr < 16; ++rr) m0 = fmaxf(m0, sacc[rr]);
        mref = max_with_partner(m0) * scale_log2;
      }
      weights();
      if (__ballot(!(ps <= kCap))) {
        float mloc = sacc[0];
#pragma unroll
        for (int rr = 1; rr < 16; ++rr) mloc = fmaxf(mloc, sacc[rr]);
        mloc = max_with_partner(mloc);
        const float mnew = fmaxf(mref, mloc * scale_log2);
        const float alpha = fast_exp2(mref - mnew);
        lsum *= alpha;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) acc[cb][rr] *= alpha;
        mref = mnew;
        weights();
      }
      lsum += ps;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[cb] = mfma32(as_bf16x8(vpre[cb]), pb0, acc[cb]);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        constexpr int kRow = kD * 2;   // bytes per V row
        const int o0 = voff[cb] + (sub * 32 + 16) * kRow;
        const u32x2 lo = lds_read_tr(reinterpret_cast<const uint16_t *>(vbase + o0));
        const u32x2 hi = lds_read_tr(reinterpret_cast<const uint16_t *>(vbase + o0 + 8 * kRow));
        const u32x4 vraw = {lo[0], lo[1], hi[0], hi[1]};
        acc[cb] = mfma32(as_bf16x8(vraw), pb1, acc[cb]);
      }
    }
    if (last) {
      // partial output of this (query, head) for block b; stored before the
      // barrier's wait, so the stores are done when the next item starts
      const bool act = qraw >= 0 && qraw < n_q;
      const float ltot = sum_with_partner(lsum);
      if (act) {
        const int64_t n_idx = inf.nb0 + tl;
        if (n_idx >= 0 && n_idx < n_part)
          put_partial(part_o, part_le, n_idx, g, hq, G, hl, h, acc, mref, ltot);
      }
    }
    async_wait_barrier();
    if (!last) {
      ++ci;
      return true;
    }
    if (!has_next) return false;
    w = wn;
    g = gn;
    inf = infn;
    qraw = qrawn;
    wn = w + per;
    has_next = wn < w_end;
    gn = gnn;
    infn = infnn;
    qrawn = qrawnn;
    nkeys = kv_keys(inf);
    kvo = kv_off(inf, g);
    n_chunks = (nkeys + kKA - 1) / kKA;
    ci = 0;
    read_q(qraw, qf);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) acc[cb][rr] = 0.f;
    mref = -INFINITY;
    lsum = 0.f;
    return true;
  };

  for (;;) {
    if (!step(std::integral_constant<int, 0>{})) break;
    if (!step(std::integral_constant<int, 1>{})) break;
  }
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

template <int G, int NB, int NW>
hipError_t launch_mfma_g(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const KvMap &kvm, const SeqTab &tab, int hq, int hkv,
                         const int32_t *sel, int topk, const int32_t *row_ptr,
                         const int32_t *q_list, const int32_t *slot, float scale, float *o,
                         float *lse, int32_t *tile_ptr, TileMeta *info, int32_t *tq,
                         uint16_t *part_o, float2 *part_le, int64_t n_part,
                         int64_t max_tiles, hipStream_t st) {
  constexpr int TPT = NW * NB * (32 / G);
  const int64_t nb = tab.blk0[tab.n];
  const float sl2 = scale * kLog2e;
  if (n_part > 0) {
    hipLaunchKernelGGL(prefill_tiles, dim3(1), dim3(1024), 0, st, row_ptr, tab, TPT,
                       max_tiles, tile_ptr);
    hipLaunchKernelGGL((prefill_tile_info<TPT>), dim3((unsigned)nb), dim3(256), 0, st,
                       row_ptr, tile_ptr, q_list, tab, kvm, info, tq);
    const int grid = 8 * ((num_cus() + 7) / 8);
    hipLaunchKernelGGL((prefill_nonown_persistent<G, NW>), dim3(grid), dim3(64 * NW),
                       0, st, q, k, v, kvm, tab, hq, hkv, tile_ptr, info, tq, sl2,
                       part_o, part_le, n_part);
  }
  // own-block pass: 4-wave workgroups (see prefill_mfma_kernel), one per
  // tile of TPTB own tokens of every query-holding block of every sequence
  constexpr int NWB = 4;
  constexpr int TPTB = NWB * NB * (32 / G);
  const int64_t tiles = (int64_t)tab.ob0[tab.n] * ((tab.B + TPTB - 1) / TPTB);
  if (tiles > 0)
    hipLaunchKernelGGL((prefill_mfma_kernel<G, NB, NWB>), dim3((unsigned)tiles, hkv),
                       dim3(64 * NWB), 0, st, q, k, v, kvm, tab, hq, sel, topk, slot,
                       sl2, part_o, part_le, n_part, o, lse);
  return hipGetLastError();
}

// Workspace of one chain on the matrix-core path: the tile table, one fp16
// partial record (+ (lse, exponent)) per (non-own pair, query head), and the
// per-tile metadata, bounded for any head group (tiles <= pairs / 16 + blocks,
// tile rows <= pairs + 256 blocks).
int64_t chain_nonown_pairs(const SeqTab &tab, int32_t topk) {
  int64_t np = 0;
  for (int s = 0; s < tab.n; ++s) np += nonown_pairs(tab.q_pos0[s], seq_nq(tab, s), tab.B, topk);
  return np;
}

struct MfmaLayout {
  size_t tile_ptr, part_o, part_le, info, tq, total;
  int64_t np, nb, max_tiles;
};
MfmaLayout mfma_layout(const SeqTab &tab, int32_t hq, int32_t d, int32_t topk, int tpt) {
  MfmaLayout L;
  L.nb = tab.blk0[tab.n];
  L.np = chain_nonown_pairs(tab, topk);
  size_t off = 0;
  L.tile_ptr = off; off += align256((size_t)(L.nb + 1) * 4);
  L.part_o = off;   off += align256((size_t)L.np * hq * d * 2);
  L.part_le = off;  off += align256((size_t)L.np * hq * 8);
  L.info = off;     off += align256((size_t)(L.np / 16 + L.nb) * sizeof(TileMeta));
  L.tq = off;       off += align256((size_t)(L.np + 256 * L.nb) * 4);
  L.total = off;
  const int64_t by_info = L.np / 16 + L.nb, by_tq = (L.np + 256 * L.nb) / tpt;
  L.max_tiles = by_info < by_tq ? by_info : by_tq;
  return L;
}

}  // namespace

bool mfma_prefill_supported(int32_t dtype, int32_t d, int32_t group) {
  return dtype == 1 && d == kD &&
         (group == 1 || group == 2 || group == 4 || group == 8 || group == 16);
}

size_t prefill_chain_ws_bytes(const SeqTab &tab, int32_t hq, int32_t d, int32_t topk) {
  return mfma_layout(tab, hq, d, topk, 16).total;
}

hipError_t launch_prefill_chain(const void *q, const void *k, const void *v,
                                const KvMap &kvm, const SeqTab &tab, int32_t hq,
                                int32_t hkv, int32_t d, const int32_t *sel, int32_t topk,
                                const int32_t *row_ptr, const int32_t *q_list,
                                const int32_t *slot, float scale, float *o, float *lse,
                                void *ws, hipStream_t st) {
  const int G = hq / hkv;
  const MfmaLayout L = mfma_layout(tab, hq, d, topk, 32 / G * 8);
  char *w = static_cast<char *>(ws);
  int32_t *tile_ptr = reinterpret_cast<int32_t *>(w + L.tile_ptr);
  uint16_t *part_o = reinterpret_cast<uint16_t *>(w + L.part_o);
  float2 *part_le = reinterpret_cast<float2 *>(w + L.part_le);
  TileMeta *info = reinterpret_cast<TileMeta *>(w + L.info);
  int32_t *tq = reinterpret_cast<int32_t *>(w + L.tq);
  const uint16_t *qq = static_cast<const uint16_t *>(q);
  const uint16_t *kk = static_cast<const uint16_t *>(k);
  const uint16_t *vv = static_cast<const uint16_t *>(v);
#define MSA_MF(GG)                                                                \
  case GG:                                                                        \
    return launch_mfma_g<GG, 1, 8>(qq, kk, vv, kvm, tab, hq, hkv, sel, topk,        \
                                   row_ptr, q_list, slot, scale, o, lse, tile_ptr,  \
                                   info, tq, part_o, part_le, L.np, L.max_tiles, st);
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

hipError_t launch_prefill_mfma(const void *q, const void *k, const void *v,
                               int64_t kv_stride, int64_t q_pos0, int64_t n_q,
                               int32_t hq, int32_t hkv, int32_t d,
                               int32_t block, const int32_t *sel, int32_t topk,
                               const int32_t *row_ptr, const int32_t *q_list,
                               const int32_t *slot, float scale, float *o,
                               float *lse, void *ws, hipStream_t st) {
  const KvMap kvm{nullptr, 0, kv_stride, 0, hkv};
  return launch_prefill_chain(q, k, v, kvm, seqtab_one(q_pos0, n_q, block), hq, hkv, d, sel,
                              topk, row_ptr, q_list, slot, scale, o, lse, ws, st);
}

hipError_t launch_prefill_paged(const void *q, const void *k_pages, const void *v_pages,
                                int64_t n_pages, const int32_t *block_table, int64_t q_pos0,
                                int64_t n_q, int32_t hq, int32_t hkv, int32_t d, int32_t block,
                                const int32_t *sel, int32_t topk, const int32_t *row_ptr,
                                const int32_t *q_list, const int32_t *slot, float scale,
                                float *o, float *lse, void *ws, hipStream_t st) {
  const KvMap kvm{block_table, n_pages, 0, 0, hkv};
  return launch_prefill_chain(q, k_pages, v_pages, kvm, seqtab_one(q_pos0, n_q, block), hq, hkv,
                              d, sel, topk, row_ptr, q_list, slot, scale, o, lse, ws, st);
}

}  // namespace msa
