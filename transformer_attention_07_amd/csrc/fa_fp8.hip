// fa_fp8.hip -- attention forward with FP8 (e4m3) inputs for MI355X (gfx950).
//
// Page "FlashAttention技术演进全景图" §5.3 lists FP8 support among the later
// versions' features; the pages give no rules for it.  Reading used here:
// q, k and v arrive as OCP e4m3 values with one fp32 descale factor per
// tensor (the real input is the stored value times its factor), and the
// operation is exactly fa_fwd's on those real inputs:
//
//     s_ij = scale * dq * dk * <q8_i, k8_j>,   O_i = dv * sum_j softmax_j(s_i.) v8_j,
//     L_i  = ln sum_j exp(s_ij)
//
// gfx950 mapping: the score product runs on the scaled FP8 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4, unit block scales), two FP8 operands
// of 32 bytes per lane: lane l of half-wave h holds row l%32 and 32 bytes of
// the head dimension starting at 64t + 32h, for the key (A, from LDS) and
// the query (B, in VGPRs) alike, so the contraction pairs the same head-dim
// elements whatever order the instruction assigns them within its slots.
// P.V stays in bf16 (v_mfma_f32_32x32x16_bf16): V's e4m3 values are widened
// exactly to bf16 while they are staged into LDS, P is rounded to bf16 as on
// the 16-bit path, and dv is applied once with the normalisation.
// Structure as fa_fwd_masked: one workgroup of four waves per (batch*head,
// 128 queries), 32 queries per wave (one per lane column), 64-key blocks of
// K (e4m3) and V (bf16) double-buffered in LDS, two workgroups per compute
// unit, online softmax per lane; causal blocks past a wave's last query are
// skipped.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "fa.h"

int fa_internal_hip_fail(hipError_t e);

#include "tiles.h"

namespace {

constexpr float kLazy = 8.0f;  // base-2 slack of the lazy exponent reference

constexpr int kQTile8 = kOwn * kWaves;  // 128 queries per workgroup
constexpr int kKBlk8 = 64;              // keys per LDS block

typedef int i32x8 __attribute__((ext_vector_type(8)));

// K block in LDS: rows of D bytes (e4m3), stride D + 16 so that the 16 rows
// of one 16-lane ds_read_b128 phase start on distinct 16-byte bank groups.
template <int D> struct K8Blk {
  static constexpr int STRIDE = D + 16;
  static constexpr int BYTES = kKBlk8 * STRIDE;
};

// 32 bytes of row r, head-dim bytes c0 .. c0+31, as an FP8 MFMA operand.
template <int D>
__device__ __forceinline__ i32x8 k8_frag(const lds_char *blk, int r, int c0) {
  const lds_char *p = blk + r * K8Blk<D>::STRIDE + c0;
  const u32x4 lo = *(const lds_u32x4 *)p;
  const u32x4 hi = *(const lds_u32x4 *)(p + 16);
  const i32x8 x = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  return x;
}

// Four e4m3 values of a word, widened exactly to bf16 (e4m3 is a subset).
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(uint32_t w) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  const u32x2 r = {Mma<__bf16>::pack2(a[0], a[1]), Mma<__bf16>::pack2(b[0], b[1])};
  return r;
}

// PAIR: 64 queries per workgroup; waves w and w + 2 hold the same 32 queries
// (group w & 1) and take alternate 32-key halves of each block, and merge
// their states at the end (the online update applied to two partial
// states).  Twice the workgroups for the same rows: for grids with fewer
// 128-row tiles than workgroup slots, whose causal tiles are few and uneven.
template <typename OT, int D, bool CAUSAL, bool PAIR>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_fp8(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ k,
    const uint8_t *__restrict__ v, OT *__restrict__ o, float *__restrict__ lse, int Nq, int Nk,
    int BH, int nqt, float c, float dv) {
  constexpr int QT = PAIR ? kQTile8 / 2 : kQTile8;  // queries per workgroup
  using M = Mma<__bf16>;
  typedef typename M::frag frag;
  constexpr int KF8 = D / 64;  // FP8 MFMAs along D for one 32x32 score block
  constexpr int NC = D / 32;   // 32-row chunks of O^T
  constexpr int KB = K8Blk<D>::BYTES;
  constexpr int VB = kKBlk8 * Blk<D>::STRIDE;  // V block, bf16 rows
  constexpr int BUF = KB + VB;
  __shared__ __attribute__((aligned(16))) char smem_raw[2 * BUF];  // [buffer][K, V]
  lds_char *smem = (lds_char *)smem_raw;

  const int bh = blockIdx.x % BH;
  // causal: the last query tiles see the most keys: first
  const int qt = CAUSAL ? nqt - 1 - (int)(blockIdx.x / BH) : (int)(blockIdx.x / BH);
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int g = lane >> 5, col = lane & 31;
  const int grp = PAIR ? (w & 1) : w;  // query group
  const int par = PAIR ? (w >> 1) : 0; // key-half parity (PAIR)
  const int q0 = qt * QT;
  const int qw0 = q0 + grp * kOwn;
  const int myq = qw0 + col;
  const uint8_t *qs = q + (size_t)bh * Nq * D;
  const uint8_t *ks = k + (size_t)bh * Nk * D;
  const uint8_t *vs = v + (size_t)bh * Nk * D;

  // Q^T fragments: 32 bytes of the lane's query per FP8 MFMA (zero past Nq)
  i32x8 qf[KF8];
#pragma unroll
  for (int t = 0; t < KF8; ++t) {
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (myq < Nq) {
      const uint8_t *p = qs + (size_t)myq * D + 64 * t + 32 * g;
      lo = *(const u32x4 *)p;
      hi = *(const u32x4 *)(p + 16);
    }
    qf[t] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  f32x16 acc[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) acc[cc] = f32x16{};
  float m = -INFINITY;
  float l = 0.f;   // this half-wave's share of the sum of p (fp32): gives L
  float lr = 0.f;  // the same sum over p as rounded for P.V: normalises O

  // staging: per 64-key block, K is 64*D bytes and V the same (widened on
  // the LDS side): 16-byte pieces, D/16 per row
  constexpr int CPR = D / 16;
  constexpr int PIECES = kKBlk8 * CPR;
  constexpr int NP = (PIECES + kThreads - 1) / kThreads;
  u32x4 rk[NP], rv[NP];
  auto gload = [&](int j0) {
#pragma unroll
    for (int n = 0; n < NP; ++n) {
      const int pc = tid + n * kThreads;
      rk[n] = rv[n] = u32x4{0u, 0u, 0u, 0u};
      const int row = j0 + pc / CPR;
      if (pc < PIECES && row < Nk) {
        const size_t off = (size_t)row * D + (pc % CPR) * 16;
        rk[n] = *(const u32x4 *)(ks + off);
        rv[n] = *(const u32x4 *)(vs + off);
      }
    }
  };
  auto sstore = [&](int buf) {
    lds_char *kb = smem + buf * BUF;
    lds_char *vb = kb + KB;
#pragma unroll
    for (int n = 0; n < NP; ++n) {
      const int pc = tid + n * kThreads;
      if (pc < PIECES) {
        const int row = pc / CPR, cb = (pc % CPR) * 16;
        *(lds_u32x4 *)(kb + row * K8Blk<D>::STRIDE + cb) = rk[n];
        // 16 e4m3 -> 16 bf16 (32 bytes) at element column cb
        const u32x2 a = e4m3x4_to_bf16(rv[n][0]), b = e4m3x4_to_bf16(rv[n][1]);
        const u32x2 e = e4m3x4_to_bf16(rv[n][2]), f = e4m3x4_to_bf16(rv[n][3]);
        lds_char *dst = vb + row * Blk<D>::STRIDE + cb * 2;
        *(lds_u32x4 *)dst = u32x4{a[0], a[1], b[0], b[1]};
        *(lds_u32x4 *)(dst + 16) = u32x4{e[0], e[1], f[0], f[1]};
      }
    }
  };

  const int kend = CAUSAL ? min(Nk, q0 + QT) : Nk;
  const int nblk = (kend + kKBlk8 - 1) / kKBlk8;
  if (nblk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int b = 0; b < nblk; ++b) {
    const int cur = b & 1;
    const bool nx = b + 1 < nblk;
    const int j0 = b * kKBlk8;
    if (nx) gload(j0 + kKBlk8);
    const lds_char *kb = smem + cur * BUF;
    const lds_char *vb = kb + KB;
#pragma unroll
    for (int hq = 0; hq < kKBlk8 / kOwn; ++hq) {
      if (PAIR && hq != par) continue;
      const int jq = j0 + hq * kOwn;
      // wave-uniform: keys past Nk, or (causal) past the wave's last query
      if (jq >= Nk || (CAUSAL && jq > qw0 + kOwn - 1)) continue;
      f32x16 s = f32x16{};
#pragma unroll
      for (int t = 0; t < KF8; ++t)
        s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            k8_frag<D>(kb, hq * kOwn + col, 64 * t + 32 * g), qf[t], s, 0, 0, 0, 127, 0, 127);
      float mx = -INFINITY;
      // wave-uniform: no key of the quarter past Nk or (causal) past the
      // wave's first query: no per-score mask
      if (jq + kOwn <= Nk && (!CAUSAL || jq + kOwn - 1 <= qw0)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[r] *= c;
          mx = fmaxf(mx, s[r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = jq + 8 * (r >> 2) + 4 * g + (r & 3);
          const bool hid = j >= Nk || (CAUSAL && j > myq);
          const float x = hid ? -INFINITY : s[r] * c;
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
        const frag pb = pack_b<__bf16>(p + 8 * tp);
        const u32x4 pw = __builtin_bit_cast(u32x4, pb);
#pragma unroll
        for (int e = 0; e < 4; ++e) lr = Mma<__bf16>::pair_sum(pw[e], lr);
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
          acc[cc] = M::mma(tr_frag<__bf16, D>(vb, hq * kOwn + 16 * tp, 32 * cc, lane), pb,
                           acc[cc]);
      }
    }
    if (nx) sstore(cur ^ 1);
    __syncthreads();
  }

  if constexpr (PAIR) {
    // merge the parity-1 wave's state into the parity-0 wave of each group
    // (the K/V buffers are free: every wave is past the loop's last barrier)
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    lds_f32x4 *x = (lds_f32x4 *)(smem + grp * ((NC * 4 + 1) * kWave * 16));
    if (par == 1) {
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          x[(cc * 4 + r4) * kWave + lane] = f32x4{acc[cc][4 * r4], acc[cc][4 * r4 + 1],
                                                  acc[cc][4 * r4 + 2], acc[cc][4 * r4 + 3]};
      x[NC * 4 * kWave + lane] = f32x4{m, l, lr, 0.f};
    }
    __syncthreads();
    if (par == 1) return;
    const f32x4 st = x[NC * 4 * kWave + lane];
    const float mn = fmaxf(m, st[0]);
    // a state with no key (m = -inf) weighs 0
    const float a0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    const float a1 = st[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st[0] - mn);
    l = l * a0 + st[1] * a1;
    lr = lr * a0 + st[2] * a1;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 y = x[(cc * 4 + r4) * kWave + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[cc][4 * r4 + e] = acc[cc][4 * r4 + e] * a0 + y[e] * a1;
      }
    m = mn;
  }
  const float lt = l + __shfl_xor(l, 32);
  const float lrt = lr + __shfl_xor(lr, 32);
  if (myq < Nq) {
    OT *os = o + (size_t)bh * Nq * D;
    // O is normalised by the rounded weights' sum, so the weights applied to
    // V sum to one (a near one-hot row then reproduces its v); L uses the
    // fp32 sum
    const float mul = lrt > 0.f ? dv / lrt : 0.f;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) store_t<OT, D>(os, myq, 32 * cc, g, acc[cc], mul);
    if (g == 0)
      lse[(size_t)bh * Nq + myq] =
          lt > 0.f ? (m + log2f(lt)) * 0.69314718055994531f : -INFINITY;
  }
}

template <typename OT, int D, bool CAUSAL, bool PAIR>
hipError_t launch_fp8_1(const void *q, const void *k, const void *v, void *o, float *lse, int Nq,
                        int Nk, int BH, float c, float dv, hipStream_t stream) {
  constexpr int QT = PAIR ? kQTile8 / 2 : kQTile8;
  const int nqt = (Nq + QT - 1) / QT;
  hipLaunchKernelGGL((fa_fwd_fp8<OT, D, CAUSAL, PAIR>), dim3((unsigned)(BH * nqt)),
                     dim3(kThreads), 0, stream, (const uint8_t *)q, (const uint8_t *)k,
                     (const uint8_t *)v, (OT *)o, lse, Nq, Nk, BH, nqt, c, dv);
  return hipGetLastError();
}

template <typename OT, int D>
hipError_t launch_fp8(const void *q, const void *k, const void *v, void *o, float *lse, int Nq,
                      int Nk, int BH, bool causal, bool pair, float c, float dv,
                      hipStream_t stream) {
  if (causal)
    return pair ? launch_fp8_1<OT, D, true, true>(q, k, v, o, lse, Nq, Nk, BH, c, dv, stream)
                : launch_fp8_1<OT, D, true, false>(q, k, v, o, lse, Nq, Nk, BH, c, dv, stream);
  return pair ? launch_fp8_1<OT, D, false, true>(q, k, v, o, lse, Nq, Nk, BH, c, dv, stream)
              : launch_fp8_1<OT, D, false, false>(q, k, v, o, lse, Nq, Nk, BH, c, dv, stream);
}

// Compute units of the current device, queried once per device (0 if the
// query fails).
int device_cus() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
  return n;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

int fa_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
               int64_t H, int64_t Nq, int64_t Nk, int64_t D, float scale, float descale_q,
               float descale_k, float descale_v, int causal, int out_f32, void *stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULLPTR;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  if (!isfinite(scale) || !isfinite(descale_q) || !isfinite(descale_k) || !isfinite(descale_v))
    return FA_ERR_SCALE;
  const float c = scale * descale_q * descale_k * 1.4426950408889634f;
  if (!isfinite(c)) return FA_ERR_SCALE;
  const int64_t lim = (int64_t)1 << 31;
  if (Nq > lim / (D * 4) - kQTile8 || Nk > lim / (D * 4) - kKBlk8) return FA_ERR_SHAPE;
  if (B > lim || H > lim || B * H > lim / ((Nq + kQTile8 - 1) / kQTile8)) return FA_ERR_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGN;
  if ((uintptr_t)lse & 3u) return FA_ERR_ALIGN;
  const int64_t BH = B * H;
  const size_t qb = (size_t)(BH * Nq * D), kb = (size_t)(BH * Nk * D);
  const size_t ob = (size_t)(BH * Nq * D) * (out_f32 ? 4 : 2), lb = (size_t)(BH * Nq) * 4;
  if (overlaps(o, ob, q, qb) || overlaps(o, ob, k, kb) || overlaps(o, ob, v, kb) ||
      overlaps(lse, lb, q, qb) || overlaps(lse, lb, k, kb) || overlaps(lse, lb, v, kb) ||
      overlaps(o, ob, lse, lb))
    return FA_ERR_OVERLAP;
  hipStream_t s = (hipStream_t)stream;
  const bool cz = causal != 0;
  // pair-split 64-query workgroups when the 128-row tiles would leave
  // workgroup slots (two per compute unit) empty
  const int cus = device_cus();
  const bool pair = cus > 0 && BH * ((Nq + kQTile8 - 1) / kQTile8) < 2 * (int64_t)cus;
  hipError_t e;
  if (out_f32)
    e = D == 64 ? launch_fp8<float, 64>(q, k, v, o, lse, (int)Nq, (int)Nk, (int)BH, cz, pair,
                                        c, descale_v, s)
                : launch_fp8<float, 128>(q, k, v, o, lse, (int)Nq, (int)Nk, (int)BH, cz, pair,
                                         c, descale_v, s);
  else
    e = D == 64 ? launch_fp8<__bf16, 64>(q, k, v, o, lse, (int)Nq, (int)Nk, (int)BH, cz, pair,
                                         c, descale_v, s)
                : launch_fp8<__bf16, 128>(q, k, v, o, lse, (int)Nq, (int)Nk, (int)BH, cz, pair,
                                          c, descale_v, s);
  if (e != hipSuccess) return fa_internal_hip_fail(e);
  return FA_OK;
}

}  // extern "C"
