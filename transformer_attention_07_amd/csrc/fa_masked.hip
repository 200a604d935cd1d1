// fa_masked.hip -- attention forward under a local-window + global-token
// mask for MI355X (gfx950, CDNA4).
//
// Page "FlashAttention-2实现与优化：高效注意力机制详解" §7 names sparse
// attention that combines local windows with global tokens as an extension
// of the tiled forward pass (and page "解释FlashAttention的显存优化原理" §二
// uses local blocks plus global key points on 100K-token sequences); the
// pages do not define the pattern.  Reading used here: key j (< Nk) is
// visible to query i iff
//
//     (causal ? 0 <= i - j < window : |i - j| < window)      local band
//  or (j < nglobal || i < nglobal) && (!causal || j <= i)     global tokens
//
// and each row is the softmax over its visible keys (the forward of
// fa_fwd restricted to them: S = scale Q K^T, running max and sum, O =
// acc / l, L = m + ln l).  A row with no visible key gets O = 0 and
// L = -inf.
//
// gfx950 mapping: one workgroup of four waves per (batch*head, 128
// queries); wave w owns 32 queries, one per lane column, with its Q
// fragments in VGPRs as MFMA B operands.  K and V stream through LDS in
// 64-key blocks (register staged, double buffered; two workgroups per
// compute unit); per 32-key half
// S^T = K Q^T (v_mfma_f32_32x32x16), the online softmax runs per lane (the
// other half of a query's keys sits in lane l ^ 32), and P^T, rounded to
// the input type, is directly the B operand of O^T += V^T P^T with V^T read
// by ds_read_b64_tr_b16.  The pattern is sparse in blocks: a workgroup
// visits only the key blocks where one of its pairs is visible, and a wave
// only the quarters where one of its own pairs is, both decided by an exact
// interval test of the three parts of the rule; hidden scores inside a
// visited quarter are -inf.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "fa.h"

int fa_internal_hip_fail(hipError_t e);

#include "tiles.h"

namespace {

constexpr float kLazy = 8.0f;  // base-2 slack of the lazy exponent reference

constexpr int kQTile = kOwn * kWaves;  // 128 queries per workgroup
// Keys per LDS block: 64 (two 32-key quarters) keep a workgroup's double-
// buffered K and V at 78 KB at D = 128, so two workgroups share a compute
// unit (two waves per SIMD) and one's loads and softmax hide behind the
// other's MFMAs.
constexpr int kMBlk = 64;

template <typename T, typename OT, int D>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_masked(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    OT *__restrict__ o, float *__restrict__ lse, int Nq, int Nk, int BH, int nqt, float c,
    Mask mk) {
  using M = Mma<T>;
  typedef typename M::frag frag;
  constexpr int KF = D / 16;
  constexpr int NC = chunks<D>();
  constexpr int BB = kMBlk * Blk<D>::STRIDE;
  __shared__ __attribute__((aligned(16))) char smem_raw[4 * BB];  // [buffer][K, V]
  lds_char *smem = (lds_char *)smem_raw;

  const int bh = blockIdx.x % BH;
  // causal: later query tiles see more keys (up to the window): first
  const int rank = blockIdx.x / BH;
  const int qt = mk.causal ? nqt - 1 - rank : rank;
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int g = lane >> 5, col = lane & 31;
  const int q0 = qt * kQTile;
  const int qw0 = q0 + w * kOwn;
  const int myq = qw0 + col;
  const int qlast = min(q0 + kQTile, Nq) - 1;     // the workgroup's last query
  const int wlast = min(qw0 + kOwn, Nq) - 1;      // the wave's last query (< qw0: none)
  const T *qs = q + (size_t)bh * Nq * D;
  const T *ks = k + (size_t)bh * Nk * D;
  const T *vs = v + (size_t)bh * Nk * D;

  frag qf[KF];
#pragma unroll
  for (int t = 0; t < KF; ++t) qf[t] = glob_frag<T, D>(qs, myq, Nq, 16 * t + 8 * g);
  f32x16 acc[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) acc[cc] = f32x16{};
  float m = -INFINITY;  // running maximum (base 2), equal in both half-waves
  float l = 0.f;   // this half-wave's share of the sum of p (fp32): gives L
  float lr = 0.f;  // the same sum over p as rounded for P.V: normalises O        // this half-wave's share of the running sum

  const int nblk = (Nk + kMBlk - 1) / kMBlk;
  auto live_block = [&](int b) {
    return mk.any(q0, qlast, b * kMBlk, min(b * kMBlk + kMBlk, Nk) - 1);
  };
  auto next_live = [&](int b) {
    while (b < nblk && !live_block(b)) ++b;
    return b;
  };
  auto kbuf = [&](int buf) { return smem + buf * 2 * BB; };

  Stage<D, kMBlk> sk, sv;
  clear_padding<D>(smem, 4 * BB, tid);
  if constexpr (D < 32) __syncthreads();
  int b = next_live(0);
  if (b < nblk) {
    sk.load(ks, b * kMBlk, Nk, tid);
    sv.load(vs, b * kMBlk, Nk, tid);
    sk.store(kbuf(0), tid);
    sv.store(kbuf(0) + BB, tid);
  }
  __syncthreads();
  int cur = 0;
  while (b < nblk) {
    const int nb = next_live(b + 1);
    const bool nx = nb < nblk;
    const int j0 = b * kMBlk;
    if (nx) {
      sk.load(ks, nb * kMBlk, Nk, tid);
      sv.load(vs, nb * kMBlk, Nk, tid);
    }
    const lds_char *kb = kbuf(cur);
    const lds_char *vb = kb + BB;
#pragma unroll 1
    for (int qq = 0; qq < kMBlk / kOwn; ++qq) {
      const int jq = j0 + qq * kOwn;
      // wave-uniform: a visible pair among this wave's queries and the quarter's keys?
      if (jq >= Nk || wlast < qw0 || !mk.any(qw0, wlast, jq, min(jq + kOwn, Nk) - 1)) continue;
      f32x16 s = f32x16{};
#pragma unroll
      for (int t = 0; t < KF; ++t)
        s = M::mma(row_frag<T, D>(kb, qq * kOwn, 16 * t, lane), qf[t], s);
      float mx = -INFINITY;
      // wave-uniform: every pair of the quarter visible (the common case
      // inside the band): no per-score mask
      if (jq + kOwn <= Nk && wlast == qw0 + kOwn - 1 &&
          mk.all(qw0, wlast, jq, jq + kOwn - 1)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[r] *= c;
          mx = fmaxf(mx, s[r]);
        }
      } else if (jq + kOwn <= Nk && qw0 >= mk.nglobal && jq >= mk.nglobal) {
        // wave-uniform: no key tail and no global row or key: the band alone
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = jq + 8 * (r >> 2) + 4 * g + (r & 3);
          const float x = mk.band(myq, j) ? s[r] * c : -INFINITY;
          s[r] = x;
          mx = fmaxf(mx, x);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = jq + 8 * (r >> 2) + 4 * g + (r & 3);
          const float x = (j < Nk && mk.visible(myq, j)) ? s[r] * c : -INFINITY;
          s[r] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // lazy reference: m moves only when a row's maximum exceeds it by more
      // than kLazy (p stays below 2^kLazy), decided for the whole wave so the
      // rescale of the accumulators is skipped together
      const bool move = mx > m + kLazy;  // also true for the first visible key
      if (__any(move)) {
        const float m_new = move ? mx : m;
        const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
        l *= alpha;
        lr *= alpha;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[cc][r] *= alpha;
        m = m_new;
      }
      // a row with no visible key yet keeps the reference 0 (p = 0)
      const float m_use = m == -INFINITY ? 0.f : m;
      float p[16];
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = __builtin_amdgcn_exp2f(s[r] - m_use);
        ps += p[r];
      }
      l += ps;
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        const frag pb = pack_b<T>(p + 8 * tp);
        const u32x4 pw = __builtin_bit_cast(u32x4, pb);
#pragma unroll
        for (int e = 0; e < 4; ++e) lr = Mma<T>::pair_sum(pw[e], lr);
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
          acc[cc] = M::mma(tr_frag<T, D>(vb, qq * kOwn + 16 * tp, 32 * cc, lane), pb, acc[cc]);
      }
    }
    if (nx) {
      sk.store(kbuf(cur ^ 1), tid);
      sv.store(kbuf(cur ^ 1) + BB, tid);
    }
    __syncthreads();
    cur ^= 1;
    b = nb;
  }

  const float lt = l + __shfl_xor(l, 32);
  const float lrt = lr + __shfl_xor(lr, 32);
  if (myq < Nq) {
    OT *os = o + (size_t)bh * Nq * D;
    // O is normalised by the rounded weights' sum, so the weights applied to
    // V sum to one (a near one-hot row then reproduces its v); L uses the
    // fp32 sum.  No visible key: O = 0
    const float inv = lrt > 0.f ? 1.f / lrt : 0.f;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) store_t<OT, D>(os, myq, 32 * cc, g, acc[cc], inv);
    if (g == 0)
      lse[(size_t)bh * Nq + myq] =
          lt > 0.f ? (m + log2f(lt)) * 0.69314718055994531f : -INFINITY;
  }
}

template <typename T, typename OT, int D>
hipError_t launch_masked(const void *q, const void *k, const void *v, void *o, float *lse,
                         int Nq, int Nk, int BH, float c, Mask mk, hipStream_t stream) {
  const int nqt = (Nq + kQTile - 1) / kQTile;
  hipLaunchKernelGGL((fa_fwd_masked<T, OT, D>), dim3((unsigned)(BH * nqt)), dim3(kThreads), 0,
                     stream, (const T *)q, (const T *)k, (const T *)v, (OT *)o, lse, Nq, Nk, BH,
                     nqt, c, mk);
  return hipGetLastError();
}

template <typename T, typename OT>
hipError_t dispatch_masked(const void *q, const void *k, const void *v, void *o, float *lse,
                           int Nq, int Nk, int BH, int D, float c, Mask mk,
                           hipStream_t stream) {
  switch (D) {
    case 16: return launch_masked<T, OT, 16>(q, k, v, o, lse, Nq, Nk, BH, c, mk, stream);
    case 32: return launch_masked<T, OT, 32>(q, k, v, o, lse, Nq, Nk, BH, c, mk, stream);
    case 64: return launch_masked<T, OT, 64>(q, k, v, o, lse, Nq, Nk, BH, c, mk, stream);
    default: return launch_masked<T, OT, 128>(q, k, v, o, lse, Nq, Nk, BH, c, mk, stream);
  }
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

int fa_fwd_masked(const void *q, const void *k, const void *v, void *o, float *lse,
                  int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, float scale,
                  int causal, int64_t window, int64_t nglobal, int dtype, void *stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULLPTR;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || window < 1 || nglobal < 0) return FA_ERR_SHAPE;
  if (D != 16 && D != 32 && D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  if (dtype != FA_BF16 && dtype != FA_BF16_OF32 && dtype != FA_F16 && dtype != FA_F16_OF32)
    return FA_ERR_DTYPE;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const int64_t lim = (int64_t)1 << 31;
  if (Nq > lim / (D * 4) - kBlk || Nk > lim / (D * 4) - kBlk) return FA_ERR_SHAPE;
  if (B > lim || H > lim || B * H > lim / ((Nq + kQTile - 1) / kQTile)) return FA_ERR_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGN;
  if ((uintptr_t)lse & 3u) return FA_ERR_ALIGN;
  const int64_t BH = B * H;
  const size_t osz = (dtype == FA_BF16_OF32 || dtype == FA_F16_OF32) ? 4 : 2;
  const size_t qb = (size_t)(BH * Nq * D) * 2, kb = (size_t)(BH * Nk * D) * 2;
  const size_t ob = (size_t)(BH * Nq * D) * osz, lb = (size_t)(BH * Nq) * 4;
  if (overlaps(o, ob, q, qb) || overlaps(o, ob, k, kb) || overlaps(o, ob, v, kb) ||
      overlaps(lse, lb, q, qb) || overlaps(lse, lb, k, kb) || overlaps(lse, lb, v, kb) ||
      overlaps(o, ob, lse, lb))
    return FA_ERR_OVERLAP;
  Mask mk;
  mk.causal = causal != 0;
  // a window of max(Nq, Nk) already covers every |i - j|; the clamp keeps
  // the band test's unsigned arithmetic exact
  const int64_t wmax = Nq > Nk ? Nq : Nk;
  mk.window = (int)(window < wmax ? window : wmax);
  mk.nglobal = (int)(nglobal < lim ? nglobal : lim - 1);
  const float c = scale * kLog2e;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  switch (dtype) {
    case FA_BF16: e = dispatch_masked<__bf16, __bf16>(q, k, v, o, lse, (int)Nq, (int)Nk, (int)BH, (int)D, c, mk, s); break;
    case FA_BF16_OF32: e = dispatch_masked<__bf16, float>(q, k, v, o, lse, (int)Nq, (int)Nk, (int)BH, (int)D, c, mk, s); break;
    case FA_F16: e = dispatch_masked<_Float16, _Float16>(q, k, v, o, lse, (int)Nq, (int)Nk, (int)BH, (int)D, c, mk, s); break;
    default: e = dispatch_masked<_Float16, float>(q, k, v, o, lse, (int)Nq, (int)Nk, (int)BH, (int)D, c, mk, s); break;
  }
  if (e != hipSuccess) return fa_internal_hip_fail(e);
  return FA_OK;
}

}  // extern "C"
