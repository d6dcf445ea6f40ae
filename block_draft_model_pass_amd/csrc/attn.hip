// Non-causal GQA block attention of the drafter (Strata PR #1426 page,
// "Target feature taps": non-causal block attention, scale 1/16; "Drafter
// runtime": 24 Q / 2 KV heads of 256; "Current limitations": 32768-cell
// window).  Every block row attends to the visible context cells
// [max(0, p - window), p) of the fp16 ring and to all block rows.
//
// Work split: one block per (KV head, chunk of 32-cell blocks); the last
// chunk holds the block rows' own keys.  Each wave owns one tile of 16 query
// rows (the 12 query heads of the KV head x block rows, packed) and keeps
// O^T [256][16] in 16 MFMA accumulators.  Per 32 cells:
//   S^T = K Q^T  : 2 cell tiles x 8 k-steps of MFMA 16x16x32 f16; the lane
//                  holding S^T[4g+i][n] and S^T[16+4g+i][n] owns exactly the
//                  8 probabilities it must feed as the B operand of P V,
//   O^T += V^T P^T: 16 MFMAs; V is stored transposed in 32-cell blocks
//                  ([block][dim][cell]) so the A operand is two 8-byte loads
//                  per lane and a block's values are one contiguous run.
// No LDS, no transposes.  A second kernel merges the chunks' (max, sum, O)
// partials flash-decoding style.
#include "common.h"

namespace dfl {

namespace {

constexpr float NEG_INF = -__builtin_huge_valf();

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  return static_cast<uint32_t>(f32_to_f16_bits(a)) |
         (static_cast<uint32_t>(f32_to_f16_bits(b)) << 16);
}

__global__ __launch_bounds__(384) void k_attn_partial(AttnArgs a) {
  const int lane = threadIdx.x & 63, t = threadIdx.x >> 6;
  if (t >= a.nqt) return;  // no block-level synchronisation in this kernel
  const int j = blockIdx.y;
  const int c = blockIdx.x;
  const int n = lane & 15, g = lane >> 4;

  // Query operand: qrow r = t*16 + n  ->  (block row r / 12, head 12 j + r % 12).
  const int r = t * 16 + n;
  const bool qv = r < G * a.B;
  const int bi = qv ? r / G : 0, hl = qv ? r % G : 0;
  const uint16_t* qp = a.q16 + (static_cast<size_t>(bi) * NQ + j * G + hl) * D;
  uint4 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qf[s] = qv ? *reinterpret_cast<const uint4*>(qp + 32 * s + 8 * g) : make_uint4(0, 0, 0, 0);

  const uint16_t *kb, *vb;
  int nblk;
  int64_t lo, hi, pstart;
  int cap;
  if (c < a.nch) {
    kb = a.ring_k + static_cast<size_t>(j) * a.cap * D;
    vb = a.ring_vt + static_cast<size_t>(j) * D * a.cap;
    cap = a.cap;
    const int blk0 = c * a.cb;
    nblk = min(a.cb, a.nb - blk0);
    pstart = a.p0 + 32 * static_cast<int64_t>(blk0);
    lo = a.lo;
    hi = a.hi;
  } else {
    kb = a.kblk + static_cast<size_t>(j) * BLK_CELLS * D;
    vb = a.vblkT + static_cast<size_t>(j) * D * BLK_CELLS;
    cap = BLK_CELLS;
    nblk = 1;
    pstart = 0;
    lo = 0;
    hi = a.B;
  }

  float m = NEG_INF, lsum = 0.f;
  f32x4 o[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ib = 0; ib < nblk; ++ib) {
    const int64_t pb = pstart + 32 * static_cast<int64_t>(ib);
    const int cidx = static_cast<int>(pb % cap);  // 32 consecutive ring cells
    const uint16_t* k0 = kb + static_cast<size_t>(cidx + n) * D + 8 * g;
    const uint16_t* k1 = k0 + 16 * D;
    // Issue the block's K loads and the first half of its V loads together
    // so the V latency hides behind the score MFMAs and the softmax; the
    // second V half is issued once the K registers are free.
    const uint16_t* vbase = vb + static_cast<size_t>(cidx / 32) * (D * 32) + n * 32 + 4 * g;
    uint4 kr0[8], kr1[8];
    uint2 va0[8], va1[8], vb0[8], vb1[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      kr0[s] = *reinterpret_cast<const uint4*>(k0 + 32 * s);
      kr1[s] = *reinterpret_cast<const uint4*>(k1 + 32 * s);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint16_t* vp = vbase + 16 * dt * 32;
      va0[dt] = *reinterpret_cast<const uint2*>(vp);
      va1[dt] = *reinterpret_cast<const uint2*>(vp + 16);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      s0 = mfma_f16(kr0[s], qf[s], s0);
      s1 = mfma_f16(kr1[s], qf[s], s1);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint16_t* vp = vbase + 16 * (dt + 8) * 32;
      vb0[dt] = *reinterpret_cast<const uint2*>(vp);
      vb1[dt] = *reinterpret_cast<const uint2*>(vp + 16);
    }
    const bool full = pb >= lo && pb + 32 <= hi;
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = s0[i] * a.scale_log2;
      x[4 + i] = s1[i] * a.scale_log2;
    }
    bool ok[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t q0 = pb + 4 * g + i, q1 = q0 + 16;
      ok[i] = full || (q0 >= lo && q0 < hi);
      ok[4 + i] = full || (q1 >= lo && q1 < hi);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = ok[i] ? x[i] : NEG_INF;
    float bm = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) bm = fmaxf(bm, x[i]);
    bm = group4_max(bm);
    const float mnew = fmaxf(m, bm);
    const float muse = mnew == NEG_INF ? 0.f : mnew;
    const float alpha = exp2f(m - muse);
    float pr[8], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr[i] = exp2f(x[i] - muse);
      ps += pr[i];
    }
    lsum = lsum * alpha + ps;
    m = mnew;
    const uint4 pf = make_uint4(pack_h2(pr[0], pr[1]), pack_h2(pr[2], pr[3]),
                                pack_h2(pr[4], pr[5]), pack_h2(pr[6], pr[7]));
    // masks for the value halves of this lane's 8 cells
    uint32_t vm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vm[i] = (ok[2 * i] ? 0x0000ffffu : 0u) | (ok[2 * i + 1] ? 0xffff0000u : 0u);
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      o[dt] *= alpha;
      const uint2 x0 = dt < 8 ? va0[dt] : vb0[dt - 8];
      const uint2 x1 = dt < 8 ? va1[dt] : vb1[dt - 8];
      const uint4 v = make_uint4(x0.x & vm[0], x0.y & vm[1], x1.x & vm[2], x1.y & vm[3]);
      o[dt] = mfma_f16(v, pf, o[dt]);
    }
  }

  lsum = group4_sum(lsum);
  const size_t base = (static_cast<size_t>(j) * (a.nch + 1) + c) * a.nqt + t;
  if (g == 0) {
    a.pm[base * 16 + n] = m;
    a.pl[base * 16 + n] = lsum;
  }
  float* op = a.po + (base * 16 + n) * D + 4 * g;
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) *reinterpret_cast<f32x4*>(op + 16 * dt) = o[dt];
}

// One block per (KV head, query tile, 16 head dims); thread (qrow, dim).
// Chunks are combined 16 at a time with every load of a group in flight,
// rescaling the running sum whenever the running max grows.
constexpr int MG = 16;

__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  const int id = blockIdx.x;
  const int dtile = id & 15;
  const int t = (id >> 4) % a.nqt;
  const int j = (id >> 4) / a.nqt;
  const int n = threadIdx.x >> 4, dd = threadIdx.x & 15;
  const int r = t * 16 + n;
  if (r >= G * a.B) return;
  const int d = dtile * 16 + dd;
  const int nc = a.nch + 1;
  const size_t cstride = static_cast<size_t>(a.nqt) * 16;  // (chunk -> chunk) in rows
  const size_t row0 = (static_cast<size_t>(j) * nc * a.nqt + t) * 16 + n;
  float M = NEG_INF, lsum = 0.f, acc = 0.f;
  for (int c0 = 0; c0 < nc; c0 += MG) {
    float mv[MG], lv[MG], ov[MG];
#pragma unroll
    for (int u = 0; u < MG; ++u) {
      const int c = c0 + u;
      const size_t row = row0 + static_cast<size_t>(c) * cstride;
      const bool ok = c < nc;
      mv[u] = ok ? a.pm[row] : NEG_INF;
      lv[u] = ok ? a.pl[row] : 0.f;
      ov[u] = ok ? a.po[row * D + d] : 0.f;
    }
    float gm = M;
#pragma unroll
    for (int u = 0; u < MG; ++u) gm = fmaxf(gm, mv[u]);
    const float sc = M == NEG_INF ? 0.f : exp2f(M - gm);
    lsum *= sc;
    acc *= sc;
#pragma unroll
    for (int u = 0; u < MG; ++u) {
      const float w = exp2f(mv[u] - gm);
      lsum += lv[u] * w;
      acc += ov[u] * w;
    }
    M = gm;
  }
  const int bi = r / G, hl = r % G;
  a.o16[static_cast<size_t>(bi) * NQ * D + (j * G + hl) * D + d] = f32_to_bf16(acc / lsum);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  if (a.B < 1 || a.B > MAXB || a.nqt < 1 || a.nqt > 6) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_attn_partial, dim3(a.nch + 1, NKV), dim3(64 * a.nqt), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_merge, dim3(NKV * a.nqt * 16), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dfl
