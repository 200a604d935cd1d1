// fa_bwd.hip -- FlashAttention-2 backward pass for MI355X (gfx950, CDNA4).
//
// The method: the forward pass keeps only O and the per-row logsumexp L
// (page "FlashAttention-2实现与优化：高效注意力机制详解", §3.1, which saves
// q, k, v, o and L for the backward pass and lists it under §7); the
// backward pass recomputes the attention probabilities block by block from
// L instead of reading a stored N x N matrix (page "解释FlashAttention的显存
// 优化原理", §一.2(2), recomputation).  With the upstream gradient dO:
//
//     P_ij  = exp(scale <q_i, k_j> - L_i)      (visible pairs, else 0)
//     dV_j  = sum_i P_ij dO_i
//     dP_ij = <dO_i, v_j>
//     Dl_i  = <dO_i, O_i>                      (= sum_j P_ij dP_ij)
//     dS_ij = P_ij (dP_ij - Dl_i)
//     dQ_i  = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i
//
// Dense problems at D = 64 and 128 run on the forward's pipelined machinery
// (fa_fwd.hip: fa_bwd_dq8 / fa_bwd_dq8_stream, then fa_bwd_dkdv8 /
// fa_bwd_dkdv8_stream, with their merge kernels when a stream-K schedule
// splits tiles); the dQ kernel there forms Dl itself.  Every other case
// (head dims 16 and 32, the masked and variable-length passes) runs the
// three kernels of this file, enqueued in order on the caller's stream:
//   * fa_bwd_prep: Dl_i = <dO_i, O_i> in fp32 into the workspace.
//   * fa_bwd_dkdv: one workgroup per (batch*head, 64 keys), 32 keys per
//     wave held in VGPRs as MFMA B operands; it streams 128-query blocks of
//     Q and dO through LDS (double-buffered, each wave taking two 32-row
//     quarters of a block) and accumulates dV^T and dK^T.
//   * fa_bwd_dq: one workgroup per (batch*head, 64 queries), 32 queries per
//     wave held in VGPRs; it streams 128-key blocks of K and V through LDS
//     and accumulates dQ^T.
// Recomputing S and dP for dQ and for dK/dV (instead of fp32 atomics on dQ)
// keeps every result deterministic and every store plain.
//
// gfx950 mapping (v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulation):
//   * dK/dV kernel: S = Q K^T and dP = dO V^T with lane l owning key l%32;
//     the accumulator registers of S and dS, rounded to the input type, are
//     directly the B operands of dV^T += dO^T P and dK^T += Q^T dS (the
//     contraction index, queries, is permuted identically on both sides), so
//     P never leaves registers.  dO^T and Q^T fragments come from
//     ds_read_b64_tr_b16 (lane L of a 16-lane group receives four
//     consecutive rows of column d0 + L).
//   * dQ kernel: S^T = K Q^T and dP^T = V dO^T with lane l owning query l%32
//     (so L_i and Dl_i are per-lane scalars); dQ^T += K^T dS^T with K^T from
//     the same transpose read.
//   * Causal: a wave skips (wave-uniformly) every block in which no pair is
//     visible; blocks on the diagonal and past Nq / Nk are masked by setting
//     P to 0.  Rows past Nq get L = +inf (P = 0), rows past Nk read as zero
//     and are never stored.
//   * Exponentials in base 2: P = 2^(c <q, k> - L log2 e), c = scale log2 e;
//     the scale of dQ and dK is applied once, in fp32, at the store.

#include <hip/hip_runtime.h>
#include <type_traits>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "fa.h"

// Records the runtime's text for fa_last_hip_error (defined with the
// forward pass's host code) and returns FA_ERR_HIP.
int fa_internal_hip_fail(hipError_t e);
// dQ on the forward's pipelined machinery (fa_fwd.hip): dense problems, D = 64
// or 128; returns false for any other case, which the kernel below takes.
// It forms Dl from O and dO itself and writes it to dl (no fa_bwd_prep).
// ws / ws_bytes: scratch for the stream schedule's partial sums (its size
// from fa_internal_dq8_bytes; with less, one workgroup per query tile).
// mask3: the local-window + global-token rule as {causal, window, nglobal}
// (one workgroup per tile over its key list), or null.
bool fa_internal_bwd_dq8(const void *q, const void *k, const void *v, const void *o,
                         const void *dout, const float *lse, float *dl, void *dq, int Nq, int Nk,
                         int BH, int D, int dtype, bool causal, float c, float scale, void *ws,
                         size_t ws_bytes, const int *mask3, void *stream, hipError_t *err);
size_t fa_internal_dq8_bytes(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, bool causal);
// dK and dV on the same machinery (fa_fwd.hip), same cases; false otherwise.
// Below two key tiles per compute unit it needs the stream schedule's
// partial sums in ws (fa_internal_dkv8_bytes); without them, false.
bool fa_internal_bwd_dkdv8(const void *q, const void *k, const void *v, const void *dout,
                           const float *lse, const float *dl, void *dk, void *dv, int Nq, int Nk,
                           int BH, int D, int dtype, bool causal, float c, float scale, void *ws,
                           size_t ws_bytes, const int *mask3, void *stream, hipError_t *err);
size_t fa_internal_dkv8_bytes(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, bool causal);
// Under the window rule mask3 the key tiles that hold global keys are cut
// into parts whose partial sums go to ws (this many bytes; with less ws
// they run whole).
size_t fa_internal_masked_dkv8_bytes(int64_t BH, int64_t Nq, int64_t Nk, int64_t D,
                                     const int *mask3);

#include "tiles.h"

namespace {

constexpr int kQBlk = 64;  // keys per LDS block of the dQ kernel

// ---------------------------------------------------------------------------
// Dl_i = <dO_i, O_i>, fp32, one row per D/8 lanes.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void fa_bwd_prep(const T *__restrict__ o,
                                                        const T *__restrict__ dout,
                                                        float *__restrict__ dl, int64_t rows) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kThreads / LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *(const u32x4 *)(o + row * D + part * 8);
    const u32x4 b = *(const u32x4 *)(dout + row * D + part * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x2 x = Mma<T>::unpack2(a[w]), y = Mma<T>::unpack2(b[w]);
      acc = fmaf(x[0], y[0], acc);
      acc = fmaf(x[1], y[1], acc);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (part == 0 && row < rows) dl[row] = acc;
}

// ---------------------------------------------------------------------------
// Sum of the two parity halves of a workgroup's accumulators: waves with
// par = 1 leave theirs in LDS, waves with par = 0 add them.  `buf` must be
// free (every wave past the last barrier of the main loop).
template <int N>
__device__ __forceinline__ void pair_sum(f32x16 (&acc)[N], lds_char *buf, int grp, int par,
                                         int lane) {
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  lds_f32x4 *x = (lds_f32x4 *)(buf + grp * (N * 16 * 4 * kWave));
  if (par == 1) {
#pragma unroll
    for (int n = 0; n < N; ++n)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        x[(n * 4 + r4) * kWave + lane] =
            f32x4{acc[n][4 * r4], acc[n][4 * r4 + 1], acc[n][4 * r4 + 2], acc[n][4 * r4 + 3]};
  }
  __syncthreads();
  if (par == 0) {
#pragma unroll
    for (int n = 0; n < N; ++n)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 y = x[(n * 4 + r4) * kWave + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[n][4 * r4 + e] += y[e];
      }
  }
}

// The (batch*head) slice, or (head, sequence) slice of a variable-length
// batch, that a workgroup works on, and its tile index.
struct Slice {
  size_t qrow, krow;  // first row of the slice in the [.., D] tensors
  int Nq, Nk, tile;
};

// Dense: workgroup id = tile rank * BH + bh.  Variable length (cu_q != 0):
// id = tile rank * (H*S) + ((h*S + s - rank) mod H*S) over [H, T, D]
// tensors, sequence s at
// rows cu[s] .. cu[s+1] (offsets clamped to [0, T]).  `rank_to_tile`
// reverses the rank order when `reverse` (ntiles tiles per slice).
__device__ __forceinline__ Slice resolve(int BH, int Nq, int Nk, const int *cu_q,
                                         const int *cu_k, int S, bool reverse, int ntiles) {
  Slice sl;
  const int id = blockIdx.x;
  if (cu_q == nullptr) {
    const int bh = id % BH, rank = id / BH;
    sl.qrow = (size_t)bh * Nq;
    sl.krow = (size_t)bh * Nk;
    sl.Nq = Nq;
    sl.Nk = Nk;
    sl.tile = reverse ? ntiles - 1 - rank : rank;
  } else {
    // BH = H, Nq = Tq, Nk = Tk.  The slice index is rotated by the rank so
    // that one sequence's tiles are spread over the XCDs (workgroup ids are
    // dealt to the 8 XCDs round robin; unrotated, H*S a multiple of 8 keeps
    // every sequence on one XCD, and the longest sequence bounds the time)
    const int rank = id / (BH * S), hs = (id % (BH * S) + rank) % (BH * S);
    const int h = hs / S, sq = hs % S;
    const int qa = max(0, min(cu_q[sq], Nq)), qb = max(qa, min(cu_q[sq + 1], Nq));
    const int ka = max(0, min(cu_k[sq], Nk)), kb = max(ka, min(cu_k[sq + 1], Nk));
    sl.qrow = (size_t)h * Nq + qa;
    sl.krow = (size_t)h * Nk + ka;
    sl.Nq = qb - qa;
    sl.Nk = kb - ka;
    sl.tile = reverse ? ntiles - 1 - rank : rank;
  }
  return sl;
}

// Rows [from, n) of a [rows, D] slice set to NaN: the rows of a
// variable-length sequence past the last tile its grid covers (the sequence
// is longer than the caller's bound), so that no row is left unwritten.
template <typename OT, int D>
__device__ __forceinline__ void nan_rows(OT *base, int from, int n) {
  const float nan = __builtin_nanf("");
  for (int i = from * D + (int)threadIdx.x; i < n * D; i += kThreads) base[i] = (OT)nan;
}

// dK and dV: one workgroup per (batch*head, kTile keys).  Wave w owns keys
// key0 + 32*(w & 1) .. +31 and, of every 128-query block, the 32-row
// quarters par and par + 2 (par = w >> 1); the two parities are summed at
// the end.
// MASKED: the local-window + global-token mask `mk` (CAUSAL is then false
// and mk.causal carries the causal rule); query blocks, wave quarters and
// pairs the mask hides are skipped or zeroed.
template <typename T, typename OT, int D, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(kThreads) void fa_bwd_dkdv(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ dl,
    OT *__restrict__ dk, OT *__restrict__ dv, int Nq, int Nk, int BH, int nkt, float c,
    float scale, const int *__restrict__ cu_q, const int *__restrict__ cu_k, int S, Mask mk) {
  using M = Mma<T>;
  typedef typename M::frag frag;
  constexpr int KF = D / 16;  // MFMA steps along D
  constexpr int NC = chunks<D>();  // 32-row chunks of dK^T / dV^T
  constexpr int BB = Blk<D>::BYTES;
  // [buffer][Q, dO] blocks, then [buffer] L*log2(e) and Dl of the block's rows
  __shared__ __attribute__((aligned(16))) char smem_raw[4 * BB + 4 * kBlk * 4];
  lds_char *smem = (lds_char *)smem_raw;
  lds_float *stats = (lds_float *)(smem + 4 * BB);

  // causal: the lowest keys see the most queries: first
  const Slice sl = resolve(BH, Nq, Nk, cu_q, cu_k, S, false, 0);
  Nq = sl.Nq;
  Nk = sl.Nk;
  const int kt = sl.tile;
  if (kt == nkt - 1 && Nk > nkt * kTile) {  // longer than the grid (variable length)
    nan_rows<OT, D>(dk + sl.krow * D, nkt * kTile, Nk);
    nan_rows<OT, D>(dv + sl.krow * D, nkt * kTile, Nk);
  }
  if (kt * kTile >= Nk) return;  // past the slice's keys (workgroup-uniform)
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int g = lane >> 5, col = lane & 31;
  const int grp = w & 1, par = w >> 1;
  const int key0 = kt * kTile + grp * kOwn;
  const int myk = key0 + col;
  const T *qs = q + sl.qrow * D;
  const T *dos = dout + sl.qrow * D;
  const T *ks = k + sl.krow * D;
  const T *vs = v + sl.krow * D;
  const float *ls = lse + sl.qrow;
  const float *ds_ = dl + sl.qrow;

  frag kf[KF], vf[KF];
#pragma unroll
  for (int t = 0; t < KF; ++t) {
    kf[t] = glob_frag<T, D>(ks, myk, Nk, 16 * t + 8 * g);
    vf[t] = glob_frag<T, D>(vs, myk, Nk, 16 * t + 8 * g);
  }
  f32x16 dva[NC], dka[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    dva[cc] = f32x16{};
    dka[cc] = f32x16{};
  }

  // queries before the tile's first key see none of its keys
  const int qstart = CAUSAL ? kt * kTile : 0;
  const int nblk = qstart < Nq ? (Nq - qstart + kBlk - 1) / kBlk : 0;

  Stage<D> st;
  float stat = 0.f;
  auto load_stat = [&](int row0) {
    const int r = row0 + (tid & (kBlk - 1));
    if (tid < kBlk)
      stat = r < Nq ? ls[r] * kLog2e : INFINITY;  // P = 0 on rows past Nq
    else
      stat = r < Nq ? ds_[r] : 0.f;
  };
  auto qbuf = [&](int buf) { return smem + buf * 2 * BB; };
  // next query block (from bb) in which some query sees a key of the tile
  const int klo = kt * kTile, khi = min(klo + kTile, Nk) - 1;
  auto next_blk = [&](int bb) {
    if constexpr (MASKED)
      while (bb < nblk &&
             !mk.any(qstart + bb * kBlk, min(qstart + bb * kBlk + kBlk, Nq) - 1, klo, khi))
        ++bb;
    return bb;
  };

  clear_padding<D>(smem, 4 * BB, tid);
  if constexpr (D < 32) __syncthreads();
  int b = next_blk(0);
  if (b < nblk) {
    st.load(qs, qstart + b * kBlk, Nq, tid);
    st.store(qbuf(0), tid);
    st.load(dos, qstart + b * kBlk, Nq, tid);
    st.store(qbuf(0) + BB, tid);
    load_stat(qstart + b * kBlk);
    stats[tid] = stat;
  }
  __syncthreads();
  int cur = 0;
  while (b < nblk) {
    const int nb = next_blk(b + 1);
    const bool nx = nb < nblk;
    const int i0 = qstart + b * kBlk;
    const int in = qstart + nb * kBlk;
    if (nx) {
      st.load(qs, in, Nq, tid);
      load_stat(in);
    }
    // wave-uniform: does any of this wave's queries see one of its keys?
    bool live;
    if constexpr (MASKED)
      live = mk.any(i0 + kOwn * par, min(i0 + kOwn * (par + 2) + kOwn, Nq) - 1, key0,
                    min(key0 + kOwn, Nk) - 1);
    else
      live = !CAUSAL || i0 + kOwn * (par + 2) + kOwn - 1 >= key0;
    const lds_char *qb = qbuf(cur);
    const lds_char *db = qb + BB;
    const lds_float *l2 = stats + cur * 2 * kBlk;
    const lds_float *dd = l2 + kBlk;
    f32x16 s[2], dp[2];
    if (live) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int r0 = kOwn * (par + 2 * hf);
        s[hf] = f32x16{};
        dp[hf] = f32x16{};
#pragma unroll
        for (int t = 0; t < KF; ++t) {
          s[hf] = M::mma(row_frag<T, D>(qb, r0, 16 * t, lane), kf[t], s[hf]);
          dp[hf] = M::mma(row_frag<T, D>(db, r0, 16 * t, lane), vf[t], dp[hf]);
        }
      }
    }
    if (nx) {
      st.store(qbuf(cur ^ 1), tid);
      stats[(cur ^ 1) * 2 * kBlk + tid] = stat;
      st.load(dos, in, Nq, tid);
    }
    if (live) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int r0 = kOwn * (par + 2 * hf);
        float p[16], dsv[16];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int ib = r0 + 8 * r4 + 4 * g;  // block row of register 4*r4
          const f32x4 lv = *(const __attribute__((address_space(3))) f32x4 *)(l2 + ib);
          const f32x4 dv4 = *(const __attribute__((address_space(3))) f32x4 *)(dd + ib);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * r4 + e;
            float pr = __builtin_amdgcn_exp2f(fmaf(s[hf][r], c, -lv[e]));
            if constexpr (MASKED) {
              if (!mk.visible(i0 + ib + e, myk)) pr = 0.f;
            } else if (CAUSAL && myk > i0 + ib + e) {
              pr = 0.f;
            }
            p[r] = pr;
            dsv[r] = pr * (dp[hf][r] - dv4[e]);
          }
        }
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
          const frag pb = pack_b<T>(p + 8 * tp);
          const frag sb = pack_b<T>(dsv + 8 * tp);
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) {
            dva[cc] = M::mma(tr_frag<T, D>(db, r0 + 16 * tp, 32 * cc, lane), pb, dva[cc]);
            dka[cc] = M::mma(tr_frag<T, D>(qb, r0 + 16 * tp, 32 * cc, lane), sb, dka[cc]);
          }
        }
      }
    }
    if (nx) st.store(qbuf(cur ^ 1) + BB, tid);
    __syncthreads();
    cur ^= 1;
    b = nb;
  }

  pair_sum<NC>(dva, smem, grp, par, lane);
  __syncthreads();
  pair_sum<NC>(dka, smem, grp, par, lane);
  if (par == 0 && myk < Nk) {
    OT *dks = dk + sl.krow * D;
    OT *dvs = dv + sl.krow * D;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      store_t<OT, D>(dvs, myk, 32 * cc, g, dva[cc], 1.f);
      store_t<OT, D>(dks, myk, 32 * cc, g, dka[cc], scale);
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (batch*head, kTile queries).  Wave w owns queries
// qw0 + 32*(w & 1) .. +31 and, of every 64-key block, the 32-key half par
// (par = w >> 1); the two parities are summed at the end.  The 64-key
// blocks keep the LDS at 78 KB and the registers under 256 at D = 128, so
// two workgroups share a compute unit (two waves per SIMD).
template <typename T, typename OT, int D, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(kThreads, 2) void fa_bwd_dq(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ dl,
    OT *__restrict__ dq, int Nq, int Nk, int BH, int nqt, float c, float scale,
    const int *__restrict__ cu_q, const int *__restrict__ cu_k, int S, Mask mk) {
  using M = Mma<T>;
  typedef typename M::frag frag;
  constexpr int KF = D / 16;
  constexpr int NC = chunks<D>();
  constexpr int BB = kQBlk * Blk<D>::STRIDE;
  constexpr int NH = kQBlk / (2 * kOwn);  // quarters per wave and block
  // [buffer][K, V] blocks
  __shared__ __attribute__((aligned(16))) char smem_raw[4 * BB];
  lds_char *smem = (lds_char *)smem_raw;

  // causal (also a causal mask): the last query tiles see the most keys: first
  const Slice sl = resolve(BH, Nq, Nk, cu_q, cu_k, S, CAUSAL || (MASKED && mk.causal), nqt);
  Nq = sl.Nq;
  Nk = sl.Nk;
  const int qt = sl.tile;
  if (qt == nqt - 1 && Nq > nqt * kTile)  // longer than the grid (variable length)
    nan_rows<OT, D>(dq + sl.qrow * D, nqt * kTile, Nq);
  if (qt * kTile >= Nq) return;  // past the slice's queries (workgroup-uniform)
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int g = lane >> 5, col = lane & 31;
  const int grp = w & 1, par = w >> 1;
  const int qw0 = qt * kTile + grp * kOwn;
  const int myq = qw0 + col;
  const T *qs = q + sl.qrow * D;
  const T *dos = dout + sl.qrow * D;
  const T *ks = k + sl.krow * D;
  const T *vs = v + sl.krow * D;

  frag qf[KF], df[KF];
#pragma unroll
  for (int t = 0; t < KF; ++t) {
    qf[t] = glob_frag<T, D>(qs, myq, Nq, 16 * t + 8 * g);
    df[t] = glob_frag<T, D>(dos, myq, Nq, 16 * t + 8 * g);
  }
  const float l2 = myq < Nq ? lse[sl.qrow + myq] * kLog2e : INFINITY;
  const float dd = myq < Nq ? dl[sl.qrow + myq] : 0.f;
  f32x16 dqa[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) dqa[cc] = f32x16{};

  // keys past the tile's last query are hidden from all its rows
  const int kend = CAUSAL ? min(Nk, qt * kTile + kTile) : Nk;
  const int nblk = (kend + kQBlk - 1) / kQBlk;
  auto kbuf = [&](int buf) { return smem + buf * 2 * BB; };
  // next key block (from bb) holding a key that some query of the tile sees
  const int qlo = qt * kTile, qhi = min(qlo + kTile, Nq) - 1;
  auto next_blk = [&](int bb) {
    if constexpr (MASKED)
      while (bb < nblk && !mk.any(qlo, qhi, bb * kQBlk, min(bb * kQBlk + kQBlk, Nk) - 1)) ++bb;
    return bb;
  };

  Stage<D, kQBlk> st;
  clear_padding<D>(smem, 4 * BB, tid);
  if constexpr (D < 32) __syncthreads();
  int b = next_blk(0);
  st.load(ks, b * kQBlk, Nk, tid);
  st.store(kbuf(0), tid);
  st.load(vs, b * kQBlk, Nk, tid);
  st.store(kbuf(0) + BB, tid);
  __syncthreads();
  int cur = 0;
  while (b < nblk) {
    const int nb = next_blk(b + 1);
    const bool nx = nb < nblk;
    const int j0 = b * kQBlk;
    if (nx) st.load(ks, nb * kQBlk, Nk, tid);
    // wave-uniform: does any of this wave's keys reach one of its queries?
    bool live;
    if constexpr (MASKED)
      live = mk.any(qw0, min(qw0 + kOwn, Nq) - 1, j0 + kOwn * par,
                    min(j0 + kOwn * (par + 2 * (NH - 1)) + kOwn, Nk) - 1);
    else
      live = !CAUSAL || j0 + kOwn * par <= qw0 + kOwn - 1;
    const lds_char *kb = kbuf(cur);
    const lds_char *vb = kb + BB;
    f32x16 s[NH], dp[NH];
    if (live) {
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        const int r0 = kOwn * (par + 2 * hf);
        s[hf] = f32x16{};
        dp[hf] = f32x16{};
#pragma unroll
        for (int t = 0; t < KF; ++t) {
          s[hf] = M::mma(row_frag<T, D>(kb, r0, 16 * t, lane), qf[t], s[hf]);
          dp[hf] = M::mma(row_frag<T, D>(vb, r0, 16 * t, lane), df[t], dp[hf]);
        }
      }
    }
    if (nx) {
      st.store(kbuf(cur ^ 1), tid);
      st.load(vs, nb * kQBlk, Nk, tid);
    }
    if (live) {
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        const int r0 = kOwn * (par + 2 * hf);
        float dsv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + r0 + 8 * (r >> 2) + 4 * g + (r & 3);
          float pr = __builtin_amdgcn_exp2f(fmaf(s[hf][r], c, -l2));
          if constexpr (MASKED) {
            if (j >= Nk || !mk.visible(myq, j)) pr = 0.f;
          } else if (j >= Nk || (CAUSAL && j > myq)) {
            pr = 0.f;
          }
          dsv[r] = pr * (dp[hf][r] - dd);
        }
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
          const frag sb = pack_b<T>(dsv + 8 * tp);
#pragma unroll
          for (int cc = 0; cc < NC; ++cc)
            dqa[cc] = M::mma(tr_frag<T, D>(kb, r0 + 16 * tp, 32 * cc, lane), sb, dqa[cc]);
        }
      }
    }
    if (nx) st.store(kbuf(cur ^ 1) + BB, tid);
    __syncthreads();
    cur ^= 1;
    b = nb;
  }

  pair_sum<NC>(dqa, smem, grp, par, lane);
  if (par == 0 && myq < Nq) {
    OT *dqs = dq + sl.qrow * D;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) store_t<OT, D>(dqs, myq, 32 * cc, g, dqa[cc], scale);
  }
}

// ---------------------------------------------------------------------------
// Host side.

struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  float *dl;
  int Nq, Nk, BH;  // variable length: Tq, Tk, H
  float scale;
  hipStream_t stream;
  // variable length only (cu_q == nullptr otherwise)
  const int *cu_q = nullptr, *cu_k = nullptr;
  int S = 1, maxq = 0, maxk = 0;
  Mask mk = {0, 1, 0};  // local-window + global-token mask (MASKED launches)
  // partial sums of the stream schedules of dK/dV, then of dQ (dense only;
  // the kernels run one after the other, so they share it)
  void *dqws = nullptr;
  size_t dqws_bytes = 0;
};

template <typename T, typename OT, int D, bool CAUSAL, bool MASKED = false>
hipError_t launch_bwd(const BwdArgs &a) {
  const float c = a.scale * kLog2e;
  const bool vl = a.cu_q != nullptr;
  hipError_t e = hipSuccess;
  // Dense and masked problems at D = 64 and 128: dQ first, on the pipelined
  // kernel, which also writes Dl; otherwise the row terms come from
  // fa_bwd_prep and dQ from fa_bwd_dq after dK/dV.
  bool done_q = false;
  if constexpr (D == 64 || D == 128) {
    if (!vl) {
      constexpr bool of32 = std::is_same<OT, float>::value;
      constexpr int code = std::is_same<T, __bf16>::value ? (of32 ? FA_BF16_OF32 : FA_BF16)
                                                          : (of32 ? FA_F16_OF32 : FA_F16);
      const int mask3[3] = {a.mk.causal, a.mk.window, a.mk.nglobal};
      done_q = fa_internal_bwd_dq8(a.q, a.k, a.v, a.o, a.dout, a.lse, a.dl, a.dq, a.Nq, a.Nk,
                                   a.BH, D, code, CAUSAL, c, a.scale, a.dqws, a.dqws_bytes,
                                   MASKED ? mask3 : nullptr, a.stream, &e);
      if (done_q && e != hipSuccess) return e;
    }
  }
  if (!done_q) {
    const int64_t rows = (int64_t)a.BH * a.Nq;
    constexpr int RPB = kThreads / (D / 8);
    hipLaunchKernelGGL((fa_bwd_prep<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)),
                       dim3(kThreads), 0, a.stream, (const T *)a.o, (const T *)a.dout, a.dl,
                       rows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // tiles per slice, and slices per tile rank
  // (a variable-length grid has at least one key tile per slice when there
  // are keys, so that keys past a zero max_seqlen_k still get their NaN)
  int nkt = ((vl ? a.maxk : a.Nk) + kTile - 1) / kTile;
  if (vl && a.Nk > 0 && nkt < 1) nkt = 1;
  const int nqt = ((vl ? a.maxq : a.Nq) + kTile - 1) / kTile;
  const int slices = vl ? a.BH * a.S : a.BH;
  bool done_kv = false;
  if constexpr (D == 64 || D == 128) {
    if (!vl) {
      constexpr bool of32 = std::is_same<OT, float>::value;
      constexpr int code = std::is_same<T, __bf16>::value ? (of32 ? FA_BF16_OF32 : FA_BF16)
                                                          : (of32 ? FA_F16_OF32 : FA_F16);
      const int mask3[3] = {a.mk.causal, a.mk.window, a.mk.nglobal};
      done_kv = fa_internal_bwd_dkdv8(a.q, a.k, a.v, a.dout, a.lse, (const float *)a.dl, a.dk,
                                      a.dv, a.Nq, a.Nk, a.BH, D, code, CAUSAL, c, a.scale,
                                      a.dqws, a.dqws_bytes, MASKED ? mask3 : nullptr, a.stream,
                                      &e);
      if (done_kv && e != hipSuccess) return e;
    }
  }
  if (nkt > 0 && !done_kv) {
    hipLaunchKernelGGL((fa_bwd_dkdv<T, OT, D, CAUSAL, MASKED>),
                       dim3((unsigned)(slices * nkt)), dim3(kThreads), 0, a.stream,
                       (const T *)a.q, (const T *)a.k, (const T *)a.v, (const T *)a.dout,
                       a.lse, (const float *)a.dl, (OT *)a.dk, (OT *)a.dv, a.Nq, a.Nk, a.BH,
                       nkt, c, a.scale, a.cu_q, a.cu_k, a.S, a.mk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (done_q) return hipSuccess;
  hipLaunchKernelGGL((fa_bwd_dq<T, OT, D, CAUSAL, MASKED>), dim3((unsigned)(slices * nqt)),
                     dim3(kThreads), 0, a.stream, (const T *)a.q, (const T *)a.k,
                     (const T *)a.v, (const T *)a.dout, a.lse, (const float *)a.dl,
                     (OT *)a.dq, a.Nq, a.Nk, a.BH, nqt, c, a.scale, a.cu_q, a.cu_k, a.S, a.mk);
  return hipGetLastError();
}

template <typename T, typename OT>
hipError_t dispatch_bwd_masked(const BwdArgs &a, int D) {
  switch (D) {
    case 16: return launch_bwd<T, OT, 16, false, true>(a);
    case 32: return launch_bwd<T, OT, 32, false, true>(a);
    case 64: return launch_bwd<T, OT, 64, false, true>(a);
    default: return launch_bwd<T, OT, 128, false, true>(a);
  }
}

template <typename T, typename OT>
hipError_t dispatch_bwd(const BwdArgs &a, int D, bool causal) {
  switch (D) {
    case 16: return causal ? launch_bwd<T, OT, 16, true>(a) : launch_bwd<T, OT, 16, false>(a);
    case 32: return causal ? launch_bwd<T, OT, 32, true>(a) : launch_bwd<T, OT, 32, false>(a);
    case 64: return causal ? launch_bwd<T, OT, 64, true>(a) : launch_bwd<T, OT, 64, false>(a);
    default:
      return causal ? launch_bwd<T, OT, 128, true>(a) : launch_bwd<T, OT, 128, false>(a);
  }
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int check_shape(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int dtype) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  if (D != 16 && D != 32 && D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  if (dtype != FA_BF16 && dtype != FA_BF16_OF32 && dtype != FA_F16 && dtype != FA_F16_OF32)
    return FA_ERR_DTYPE;
  const int64_t lim = (int64_t)1 << 31;
  // per-slice byte offsets (fp32 gradients at most 4 bytes an element) fit in
  // 32 bits; grids are one-dimensional
  if (Nq > lim / (D * 4) - kTile || Nk > lim / (D * 4) - kTile) return FA_ERR_SHAPE;
  if (B > lim || H > lim || B * H > lim / ((Nq > Nk ? Nq : Nk) / kTile + 1)) return FA_ERR_SHAPE;
  if (B * H * Nq > lim) return FA_ERR_SHAPE;
  return FA_OK;
}

// Partial sums of the stream schedules past the row terms: the larger of
// the dK/dV and the dQ needs (the two never hold data at once).
size_t stream_bytes(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, bool causal) {
  const size_t a = fa_internal_dq8_bytes(BH, Nq, Nk, D, causal);
  const size_t b = fa_internal_dkv8_bytes(BH, Nq, Nk, D, causal);
  return a > b ? a : b;
}

}  // namespace

extern "C" {

int fa_bwd_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                          int causal, int dtype, size_t *bytes) {
  if (!bytes) return FA_ERR_NULLPTR;
  *bytes = 0;
  const int st = check_shape(B, H, Nq, Nk, D, dtype);
  if (st != FA_OK) return st;
  const size_t lb = (size_t)(B * H * Nq) * sizeof(float);
  const size_t extra = stream_bytes(B * H, Nq, Nk, D, causal != 0);
  *bytes = extra ? (lb + 255) / 256 * 256 + extra : lb;
  return FA_OK;
}

int fa_bwd_masked_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                                 int causal, int64_t window, int64_t nglobal, int dtype,
                                 size_t *bytes) {
  if (!bytes) return FA_ERR_NULLPTR;
  *bytes = 0;
  if (window < 1 || nglobal < 0) return FA_ERR_SHAPE;
  const int st = check_shape(B, H, Nq, Nk, D, dtype);
  if (st != FA_OK) return st;
  const size_t lb = (size_t)(B * H * Nq) * sizeof(float);
  const int64_t lim = (int64_t)1 << 31;
  const int mask3[3] = {causal != 0, (int)(window < lim ? window : lim - 1),
                        (int)(nglobal < lim ? nglobal : lim - 1)};
  const size_t extra = fa_internal_masked_dkv8_bytes(B * H, Nq, Nk, D, mask3);
  *bytes = extra ? (lb + 255) / 256 * 256 + extra : lb;
  return FA_OK;
}

static int bwd_dense(const void *q, const void *k, const void *v, const void *o,
                     const float *lse, const void *dout, void *dq, void *dk, void *dv,
                     int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, float scale,
                     int causal, int dtype, void *workspace, size_t workspace_bytes,
                     void *stream, const Mask *mk) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULLPTR;
  int st = check_shape(B, H, Nq, Nk, D, dtype);
  if (st != FA_OK) return st;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout |
       (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv) & 15u)
    return FA_ERR_ALIGN;
  if (((uintptr_t)lse & 3u) || ((uintptr_t)workspace & 15u)) return FA_ERR_ALIGN;
  const int64_t BH = B * H;
  const size_t gsz = (dtype == FA_BF16_OF32 || dtype == FA_F16_OF32) ? 4 : 2;
  const size_t qb = (size_t)(BH * Nq * D) * 2, kb = (size_t)(BH * Nk * D) * 2;
  const size_t lb = (size_t)(BH * Nq) * 4;
  const size_t dqb = (size_t)(BH * Nq * D) * gsz, dkb = (size_t)(BH * Nk * D) * gsz;
  const size_t need = lb;
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  // past the row terms (rounded up to 256 bytes): the stream schedules'
  // partial sums, used when the workspace holds them
  const size_t off = (lb + 255) / 256 * 256;
  int mask3[3] = {0, 1, 0};
  if (mk) {
    mask3[0] = mk->causal;
    mask3[1] = mk->window;
    mask3[2] = mk->nglobal;
  }
  const size_t extra = mk ? fa_internal_masked_dkv8_bytes(BH, Nq, Nk, D, mask3)
                          : stream_bytes(BH, Nq, Nk, D, causal != 0);
  const size_t used = extra && workspace_bytes >= off + extra ? off + extra : need;
  // written buffers against every buffer of the call
  const void *outs[4] = {dq, dk, dv, workspace};
  const size_t osz[4] = {dqb, dkb, dkb, used};
  const void *ins[6] = {q, k, v, o, dout, lse};
  const size_t isz[6] = {qb, kb, kb, qb, qb, lb};
  for (int x = 0; x < 4; ++x) {
    for (int y = 0; y < 6; ++y)
      if (overlaps(outs[x], osz[x], ins[y], isz[y])) return FA_ERR_OVERLAP;
    for (int y = x + 1; y < 4; ++y)
      if (overlaps(outs[x], osz[x], outs[y], osz[y])) return FA_ERR_OVERLAP;
  }
  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dl = (float *)workspace;
  if (used > need) {
    a.dqws = (char *)workspace + off;
    a.dqws_bytes = extra;
  }
  a.Nq = (int)Nq;
  a.Nk = (int)Nk;
  a.BH = (int)BH;
  a.scale = scale;
  a.stream = (hipStream_t)stream;
  const bool cz = causal != 0;
  hipError_t e;
  if (mk) {
    a.mk = *mk;
    switch (dtype) {
      case FA_BF16: e = dispatch_bwd_masked<__bf16, __bf16>(a, (int)D); break;
      case FA_BF16_OF32: e = dispatch_bwd_masked<__bf16, float>(a, (int)D); break;
      case FA_F16: e = dispatch_bwd_masked<_Float16, _Float16>(a, (int)D); break;
      default: e = dispatch_bwd_masked<_Float16, float>(a, (int)D); break;
    }
  } else {
    switch (dtype) {
      case FA_BF16: e = dispatch_bwd<__bf16, __bf16>(a, (int)D, cz); break;
      case FA_BF16_OF32: e = dispatch_bwd<__bf16, float>(a, (int)D, cz); break;
      case FA_F16: e = dispatch_bwd<_Float16, _Float16>(a, (int)D, cz); break;
      default: e = dispatch_bwd<_Float16, float>(a, (int)D, cz); break;
    }
  }
  if (e != hipSuccess) return fa_internal_hip_fail(e);
  return FA_OK;
}

int fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
           const void *dout, void *dq, void *dk, void *dv, int64_t B, int64_t H, int64_t Nq,
           int64_t Nk, int64_t D, float scale, int causal, int dtype, void *workspace,
           size_t workspace_bytes, void *stream) {
  return bwd_dense(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, D, scale, causal, dtype,
                   workspace, workspace_bytes, stream, nullptr);
}

int fa_bwd_masked(const void *q, const void *k, const void *v, const void *o,
                  const float *lse, const void *dout, void *dq, void *dk, void *dv, int64_t B,
                  int64_t H, int64_t Nq, int64_t Nk, int64_t D, float scale, int causal,
                  int64_t window, int64_t nglobal, int dtype, void *workspace,
                  size_t workspace_bytes, void *stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULLPTR;
  if (window < 1 || nglobal < 0) return FA_ERR_SHAPE;
  const int64_t lim = (int64_t)1 << 31;
  Mask mk;
  mk.causal = causal != 0;
  mk.window = (int)(window < lim ? window : lim - 1);
  mk.nglobal = (int)(nglobal < lim ? nglobal : lim - 1);
  return bwd_dense(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, D, scale, causal, dtype,
                   workspace, workspace_bytes, stream, &mk);
}

int fa_bwd_varlen(const void *q, const void *k, const void *v, const void *o,
                  const float *lse, const void *dout, void *dq, void *dk, void *dv,
                  const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int64_t S,
                  int64_t H, int64_t Tq, int64_t Tk, int64_t max_seqlen_q,
                  int64_t max_seqlen_k, int64_t D, float scale, int causal, int dtype,
                  void *workspace, size_t workspace_bytes, void *stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !cu_seqlens_q ||
      !cu_seqlens_k)
    return FA_ERR_NULLPTR;
  if (S < 1 || H < 1 || Tq < 1 || Tk < 0 || max_seqlen_q < 1 || max_seqlen_k < 0)
    return FA_ERR_SHAPE;
  int st = check_shape(1, H, Tq, Tk > 0 ? Tk : 1, D, dtype);
  if (st != FA_OK) return st;
  if (max_seqlen_q > Tq) max_seqlen_q = Tq;
  if (max_seqlen_k > Tk) max_seqlen_k = Tk;
  const int64_t lim = (int64_t)1 << 31;
  const int64_t tiles = (max_seqlen_q > max_seqlen_k ? max_seqlen_q : max_seqlen_k) / kTile + 1;
  if (S > lim || H * S > lim / tiles) return FA_ERR_SHAPE;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout |
       (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv) & 15u)
    return FA_ERR_ALIGN;
  if (((uintptr_t)lse | (uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k) & 3u ||
      ((uintptr_t)workspace & 15u))
    return FA_ERR_ALIGN;
  const size_t gsz = (dtype == FA_BF16_OF32 || dtype == FA_F16_OF32) ? 4 : 2;
  const size_t qb = (size_t)(H * Tq * D) * 2, kb = (size_t)(H * Tk * D) * 2;
  const size_t lb = (size_t)(H * Tq) * 4, cb = (size_t)(S + 1) * 4;
  const size_t dqb = (size_t)(H * Tq * D) * gsz, dkb = (size_t)(H * Tk * D) * gsz;
  const size_t need = lb;
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  const void *outs[4] = {dq, dk, dv, workspace};
  const size_t osz[4] = {dqb, dkb, dkb, need};
  const void *ins[8] = {q, k, v, o, dout, lse, cu_seqlens_q, cu_seqlens_k};
  const size_t isz[8] = {qb, kb, kb, qb, qb, lb, cb, cb};
  for (int x = 0; x < 4; ++x) {
    for (int y = 0; y < 8; ++y)
      if (overlaps(outs[x], osz[x], ins[y], isz[y])) return FA_ERR_OVERLAP;
    for (int y = x + 1; y < 4; ++y)
      if (overlaps(outs[x], osz[x], outs[y], osz[y])) return FA_ERR_OVERLAP;
  }
  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dl = (float *)workspace;
  a.Nq = (int)Tq;
  a.Nk = (int)Tk;
  a.BH = (int)H;
  a.scale = scale;
  a.stream = (hipStream_t)stream;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.S = (int)S;
  a.maxq = (int)max_seqlen_q;
  a.maxk = (int)max_seqlen_k;
  const bool cz = causal != 0;
  hipError_t e;
  switch (dtype) {
    case FA_BF16: e = dispatch_bwd<__bf16, __bf16>(a, (int)D, cz); break;
    case FA_BF16_OF32: e = dispatch_bwd<__bf16, float>(a, (int)D, cz); break;
    case FA_F16: e = dispatch_bwd<_Float16, _Float16>(a, (int)D, cz); break;
    default: e = dispatch_bwd<_Float16, float>(a, (int)D, cz); break;
  }
  if (e != hipSuccess) return fa_internal_hip_fail(e);
  return FA_OK;
}

}  // extern "C"
