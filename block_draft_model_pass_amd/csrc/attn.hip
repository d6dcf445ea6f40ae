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
//   O^T += V^T P^T: 16 MFMAs; V is stored transposed (cell index fastest) so
//                  the A operand is two 8-byte loads per lane.
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
  int vstride, nblk;
  int64_t lo, hi, pstart;
  int cap;
  if (c < a.nch) {
    kb = a.ring_k + static_cast<size_t>(j) * a.cap * D;
    vb = a.ring_vt + static_cast<size_t>(j) * D * a.cap;
    vstride = a.cap;
    cap = a.cap;
    const int blk0 = c * a.cb;
    nblk = min(a.cb, a.nb - blk0);
    pstart = a.p0 + 32 * static_cast<int64_t>(blk0);
    lo = a.lo;
    hi = a.hi;
  } else {
    kb = a.kblk + static_cast<size_t>(j) * BLK_CELLS * D;
    vb = a.vblkT + static_cast<size_t>(j) * D * BLK_CELLS;
    vstride = BLK_CELLS;
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
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      s0 = mfma_f16(*reinterpret_cast<const uint4*>(k0 + 32 * s), qf[s], s0);
      s1 = mfma_f16(*reinterpret_cast<const uint4*>(k1 + 32 * s), qf[s], s1);
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
      const uint16_t* vp = vb + static_cast<size_t>(16 * dt + n) * vstride + cidx + 4 * g;
      uint2 v0 = *reinterpret_cast<const uint2*>(vp);
      uint2 v1 = *reinterpret_cast<const uint2*>(vp + 16);
      uint4 va = make_uint4(v0.x & vm[0], v0.y & vm[1], v1.x & vm[2], v1.y & vm[3]);
      o[dt] = mfma_f16(va, pf, o[dt]);
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

// One block per (KV head, query tile, query row); thread = head dimension.
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  const int id = blockIdx.x;
  const int n = id & 15;
  const int t = (id >> 4) % a.nqt;
  const int j = (id >> 4) / a.nqt;
  const int r = t * 16 + n;
  if (r >= G * a.B) return;
  const int bi = r / G, hl = r % G;
  const int nc = a.nch + 1;
  const int d = threadIdx.x;
  float M = NEG_INF;
  for (int c = 0; c < nc; ++c) {
    const size_t base = (static_cast<size_t>(j) * nc + c) * a.nqt + t;
    M = fmaxf(M, a.pm[base * 16 + n]);
  }
  float lsum = 0.f, acc = 0.f;
  for (int c = 0; c < nc; ++c) {
    const size_t base = (static_cast<size_t>(j) * nc + c) * a.nqt + t;
    const float w = exp2f(a.pm[base * 16 + n] - M);
    lsum += a.pl[base * 16 + n] * w;
    acc += a.po[(base * 16 + n) * D + d] * w;
  }
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
