// fa_fwd.hip -- FlashAttention-2 forward pass for MI355X (gfx950, CDNA4).
//
// The method (page "FlashAttention-2实现与优化：高效注意力机制详解", §3.1 and
// §3.2; page "解释FlashAttention的显存优化原理", §一.2): each workgroup owns a
// tile of query rows and walks the key/value sequence tile by tile.  Per key
// tile it forms the scores S = scale * Q K^T, updates a running row maximum m
// and row sum l (online softmax), rescales its fp32 output accumulator by
// exp(m_old - m_new) and adds P V.  At the end it writes O = acc / l and the
// per-row logsumexp L = m + ln l.  The score matrix lives only in registers.
//
// gfx950 mapping (one workgroup = 4 wave64s = 128 query rows, 32 per wave):
//   * S^T = K Q^T on v_mfma_f32_32x32x16_{bf16,f16} (v_mfma_f32_32x32x2_f32
//     for fp32 inputs).  Computing the transpose puts one query per lane
//     column: lane l owns query (l mod 32) and 16 of each 32-key block, so a
//     row maximum or sum is a reduction inside the lane plus one exchange with
//     lane l^32.
//   * The S^T accumulator registers, rounded to the input type, are exactly
//     the B operand of O^T += V^T P^T: no shuffle of P through LDS.
//   * K tiles sit in LDS row-major (row stride padded by 16 bytes so eight
//     consecutive rows start on distinct banks); V tiles are stored
//     transposed (V^T, row stride padded by 8 bytes) so each lane reads 4
//     consecutive keys of one head-dim column with one 8-byte LDS read.
//   * K/V tiles are double-buffered: the global loads of tile j+1 are issued
//     before the MFMAs of tile j and written to the other LDS buffer after
//     them, so one barrier per tile suffices.
//   * Ragged tails: every global read goes through a buffer resource whose
//     size is the (batch, head) slice, so rows past Nq / Nk read as zero;
//     scores of keys >= Nk are set to -inf before the softmax, and rows >= Nq
//     are never stored.
//   * Causal: key tiles past a wave's last query are skipped by that wave;
//     only tiles that straddle the diagonal (or the Nk tail) pay for masking.
//     Workgroups are issued longest-first, and consecutive workgroup ids
//     (which the dispatcher spreads over the 8 XCDs) take different heads so
//     that one head's K/V stays within one XCD's L2 when B*H is a multiple
//     of 8.
//   * The softmax works in base 2: c = scale*log2(e) is folded into the
//     scores, p = 2^(c*s - m2), and L = ln2 * (m2 + log2 l).

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "fa.h"

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per tile

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Word 3 of a gfx9 buffer resource: raw (untyped) dword access, bounds
// checked against num_records; out-of-range loads return zero.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base,
                                                           uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                           (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// ---------------------------------------------------------------------------
// 16-bit input types: one MFMA shape, two element types.
template <typename T> struct Mfma16;

template <> struct Mfma16<__bf16> {
  typedef bf16x8 frag;
  typedef bf16x4 quad;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // acc + x.lo + x.hi for a packed pair of bf16 (v_dot2c_f32_bf16 with (1,1)).
  static __device__ __forceinline__ float pair_sum(uint32_t x, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), one, acc, false);
  }
};

template <> struct Mfma16<_Float16> {
  typedef f16x8 frag;
  typedef f16x4 quad;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float pair_sum(uint32_t x, float acc) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), one, acc, false);
  }
};

// Key index (relative to its 32-key block) held by accumulator register r of
// a lane in half-wave g, for the 32x32 MFMA output layout: row
// 8*(r/4) + 4*g + (r%4), column = lane % 32.
__device__ __forceinline__ int acc_row(int r, int g) {
  return 8 * (r >> 2) + 4 * g + (r & 3);
}

struct WorkItem {
  int bh;  // flattened batch*head
  int q0;  // first query row of the workgroup
};

__device__ __forceinline__ WorkItem work_item(int BH, int nqt, bool causal) {
  const int id = blockIdx.x;
  const int bh = id % BH;
  const int t = id / BH;
  const int qt = causal ? (nqt - 1 - t) : t;
  return {bh, qt * kBM};
}

// Applies the scale (base-2 folded) and the masks to one S^T tile, in place.
template <bool CAUSAL>
__device__ __forceinline__ void scale_and_mask(f32x16 (&s)[kBN / 32], float c, int k0,
                                               int Nk, int my_q, int g,
                                               bool need_mask) {
#pragma unroll
  for (int kb = 0; kb < kBN / 32; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = s[kb][r] * c;
      if (need_mask) {
        const int key = k0 + kb * 32 + acc_row(r, g);
        const bool hidden = (key >= Nk) || (CAUSAL && key > my_q);
        x = hidden ? -INFINITY : x;
      }
      s[kb][r] = x;
    }
  }
}

// Online-softmax update of one tile (scores already scaled to base 2).
// Replaces s by p = 2^(s - m_new), returns alpha = 2^(m_old - m_new) and
// updates m (row max, identical in both half-waves) and l (this half-wave's
// partial row sum; the halves are added once, in the epilogue).
__device__ __forceinline__ float online_softmax(f32x16 (&s)[kBN / 32], float &m,
                                                float &l) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(m, mx);
  const float alpha = __builtin_amdgcn_exp2f(m - m_new);
  float psum = 0.f;
#pragma unroll
  for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(s[kb][r] - m_new);
      s[kb][r] = p;
      psum += p;
    }
  l = l * alpha + psum;
  m = m_new;
  return alpha;
}

template <typename OT>
__device__ __forceinline__ void store4(OT *dst, f32x4 v);

template <> __device__ __forceinline__ void store4<float>(float *dst, f32x4 v) {
  *reinterpret_cast<f32x4 *>(dst) = v;
}
template <> __device__ __forceinline__ void store4<__bf16>(__bf16 *dst, f32x4 v) {
  *reinterpret_cast<bf16x4 *>(dst) = __builtin_convertvector(v, bf16x4);
}
template <> __device__ __forceinline__ void store4<_Float16>(_Float16 *dst, f32x4 v) {
  *reinterpret_cast<f16x4 *>(dst) = __builtin_convertvector(v, f16x4);
}

// Writes O = acc / lo (rows < Nq) and L = ln2 * (m + log2 l).  l and lo are
// half-wave partial sums; lo is the normaliser of O (by default l itself).
template <int D, typename OT>
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[(D < 32 ? 32 : D) / 32],
                                         float m, float l, OT *o, float *lse, int bh,
                                         int Nq, int my_q, int g, float lo = -1.f) {
  const float lt = l + __shfl_xor(l, 32);
  const float lot = lo < 0.f ? lt : lo + __shfl_xor(lo, 32);
  if (my_q >= Nq) return;
  const float inv = 1.0f / lot;
  OT *orow = o + ((size_t)bh * Nq + my_q) * D;
#pragma unroll
  for (int db = 0; db < (D < 32 ? 32 : D) / 32; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = db * 32 + 8 * r4 + 4 * g;
      if (D >= 32 || d < D) {
        f32x4 v = {acc[db][4 * r4 + 0] * inv, acc[db][4 * r4 + 1] * inv,
                   acc[db][4 * r4 + 2] * inv, acc[db][4 * r4 + 3] * inv};
        store4<OT>(orow + d, v);
      }
    }
  }
  if (g == 0) lse[(size_t)bh * Nq + my_q] = (m + log2f(lt)) * 0.69314718055994531f;
}

// ---------------------------------------------------------------------------
// bf16 / fp16 inputs.
template <typename T, typename OT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fa_fwd_mfma16(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    OT *__restrict__ o, float *__restrict__ lse, int Nq, int Nk, int BH, int nqt,
    float c) {
  typedef typename Mfma16<T>::frag frag;
  constexpr int KS = D + 8;                // K row stride in LDS (elements)
  constexpr int DV = D < 32 ? 32 : D;      // V^T rows (MFMA M-blocks are 32)
  constexpr int VS = kBN + 4;              // V^T row stride in LDS (elements)
  constexpr int K_ELEMS = kBN * KS;
  constexpr int V_ELEMS = DV * VS;
  constexpr int BUF = K_ELEMS + V_ELEMS;
  constexpr int CPR = D / 8;               // 16-byte chunks per K/V row
  constexpr int NCH = kBN * CPR;           // chunks per tile
  constexpr int LPT = (NCH + kThreads - 1) / kThreads;
  constexpr int QF = D / 16;               // Q fragments (MFMA k-steps over D)
  constexpr int NDB = DV / 32;             // O^T M-blocks

  __shared__ __attribute__((aligned(16))) T smem[2 * BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const WorkItem wi = work_item(BH, nqt, CAUSAL);
  const int qw = wi.q0 + wave * 32;
  const int my_q = qw + l32;

  const size_t qoff = (size_t)wi.bh * Nq * D;
  const size_t koff = (size_t)wi.bh * Nk * D;
  const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(q + qoff, (uint32_t)Nq * D * sizeof(T));
  const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(k + koff, (uint32_t)Nk * D * sizeof(T));
  const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(v + koff, (uint32_t)Nk * D * sizeof(T));

  // Q^T fragments stay in registers for the whole key loop.
  frag qf[QF];
#pragma unroll
  for (int f = 0; f < QF; ++f) {
    const uint32_t off = ((uint32_t)my_q * D + 16 * f + 8 * g) * sizeof(T);
    qf[f] = __builtin_bit_cast(frag, load16(q_rs, off));
  }

  u32x4 kreg[LPT], vreg[LPT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int ch = tid + i * kThreads;
      if (NCH % kThreads == 0 || ch < NCH) {
        const int row = ch / CPR;
        const int col = (ch % CPR) * 8;
        const uint32_t off = ((uint32_t)(kt * kBN + row) * D + col) * sizeof(T);
        kreg[i] = load16(k_rs, off);
        vreg[i] = load16(v_rs, off);
      }
    }
  };
  auto swrite = [&](int buf) {
    T *Ks = smem + buf * BUF;
    T *Vt = Ks + K_ELEMS;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int ch = tid + i * kThreads;
      if (NCH % kThreads == 0 || ch < NCH) {
        const int row = ch / CPR;
        const int col = (ch % CPR) * 8;
        *reinterpret_cast<u32x4 *>(Ks + row * KS + col) = kreg[i];
        const frag ve = __builtin_bit_cast(frag, vreg[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) Vt[(col + e) * VS + row] = ve[e];
      }
    }
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  const int kend = CAUSAL ? min(Nk, wi.q0 + kBM) : Nk;
  const int nkt = (kend + kBN - 1) / kBN;

  gload(0);
  swrite(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) gload(kt + 1);
    const int k0 = kt * kBN;
    const bool active = !CAUSAL || (k0 <= qw + 31);
    if (active) {
      const T *Ks = smem + (kt & 1) * BUF;
      const T *Vt = Ks + K_ELEMS;
      f32x16 s[kBN / 32];
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int f = 0; f < QF; ++f) {
          const frag a =
              *reinterpret_cast<const frag *>(Ks + (kb * 32 + l32) * KS + 16 * f + 8 * g);
          s[kb] = Mfma16<T>::mma(a, qf[f], s[kb]);
        }
      }
      const bool need_mask = (k0 + kBN > Nk) || (CAUSAL && k0 + kBN - 1 > qw);
      scale_and_mask<CAUSAL>(s, c, k0, Nk, my_q, g, need_mask);
      const float alpha = online_softmax(s, m, l);
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
#pragma unroll
      for (int st = 0; st < kBN / 16; ++st) {
        const int kb = st >> 1;
        const int h = st & 1;
        const f32x8 pv = {s[kb][8 * h + 0], s[kb][8 * h + 1], s[kb][8 * h + 2],
                          s[kb][8 * h + 3], s[kb][8 * h + 4], s[kb][8 * h + 5],
                          s[kb][8 * h + 6], s[kb][8 * h + 7]};
        const frag pf = __builtin_convertvector(pv, frag);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const T *vp = Vt + (db * 32 + l32) * VS + st * 16 + 4 * g;
          const u32x2 lo = *reinterpret_cast<const u32x2 *>(vp);
          const u32x2 hi = *reinterpret_cast<const u32x2 *>(vp + 8);
          const u32x4 raw = {lo[0], lo[1], hi[0], hi[1]};
          acc[db] = Mfma16<T>::mma(__builtin_bit_cast(frag, raw), pf, acc[db]);
        }
      }
    }
    if (kt + 1 < nkt) swrite((kt + 1) & 1);
    __syncthreads();
  }

  epilogue<D, OT>(acc, m, l, o, lse, wi.bh, Nq, my_q, g);
}

// ---------------------------------------------------------------------------
// Pipelined kernel for 16-bit inputs with D = 64 or 128.
//
// Same arithmetic and register layouts as fa_fwd_mfma16; what differs:
//   * K and V tiles (64 keys) go global -> LDS directly (buffer_load ... lds,
//     16 bytes per lane, written lane-linearly) into a K ring and a V ring of
//     four stages each; nothing passes through VGPRs.  Tile t+3 of K and
//     tile t+2 of V are requested while tile t is computed on.
//   * Rows are padded in LDS: K rows to 17 16-byte slots (9 for D=64) so the
//     16 rows read by one ds_read_b128 pass start on distinct bank groups; V
//     rows to 20 slots (12 for D=64), where the transpose reads below are
//     fastest.  Padding slots are loaded from an out-of-range offset (zero, no
//     memory traffic).  With fixed strides every fragment address is a
//     per-lane base plus an immediate.
//   * V^T fragments come from ds_read_b64_tr_b16: within each 16-lane group,
//     lane s points at V[k0 + s/4][d0 + 4*(s%4)] and lane L receives
//     V[k0..k0+3][d0 + L], i.e. four consecutive keys of one column.
//   * The arithmetic is pipelined over 32-key blocks: sub-step b issues the
//     P.V MFMAs of block b-1 and the K.Q^T MFMAs of block b+1 beside the
//     softmax of block b, so the MFMA pipe and the VALU work side by side.
//     With 32-row waves the causal diagonal is exactly block qw/32 of each
//     wave; it alone is masked, later blocks are skipped.
//   * The running maximum used as the exponent reference only moves when some
//     row's maximum exceeds it by more than kLazy (base-2 units; a
//     wave-uniform decision), so the accumulator is rarely rescaled; p stays
//     below 2^kLazy and O = acc / l is unchanged.
//   * Half-wave maxima are exchanged with v_permlane32_swap.
//   * A negative scale is applied by flipping the sign bits of the Q
//     fragments once (exact), so the folded factor c is never negative.

constexpr float kLazy = 8.0f;
constexpr uint32_t kOutOfRange = 0x40000000u;  // > any slice size (checked on the host)
constexpr int kStages = 4;

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ u32x2 read_tr16(const lds_char *p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
  return __builtin_bit_cast(u32x2, r);
}

// s_waitcnt vmcnt(N) (gfx9 encoding); with LGKM0 also lgkmcnt(0).
template <int N, bool LGKM0 = false>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) |
                             (LGKM0 ? 0 : (0xF << 8)));
}

// Workgroup barrier for the DMA ring.  Waits until at most N of this wave's
// buffer loads are in flight and all of its LDS reads have returned, then
// meets the other waves.  No memory fence: a workgroup fence would wait for
// every load in flight (vmcnt(0)) and drain the ring.  The empty asm
// statements keep the compiler from moving LDS accesses across.
template <int N>
__device__ __forceinline__ void ring_barrier() {
  wait_vmcnt<N, true>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <typename T, int D>
struct PipeLayout {
  static constexpr int C = D / 8;                     // 16-byte chunks per row
  static constexpr int SK = D == 128 ? 17 : 9;        // K row stride (slots)
  static constexpr int SV = D == 128 ? 20 : 12;       // V row stride (slots)
  static constexpr int K_BYTES = kBN * SK * 16;
  static constexpr int V_BYTES = kBN * SV * 16;
  static constexpr int K_INS = kBN * SK / kWave;      // DMA instructions per K tile
  static constexpr int V_INS = kBN * SV / kWave;
  static constexpr int K_PER_WAVE = (K_INS + kWaves - 1) / kWaves;  // wave 0's share
  static constexpr int V_PER_WAVE = V_INS / kWaves;
  static constexpr int K_EXTRA = K_INS % kWaves;      // waves < K_EXTRA issue one more
  static constexpr int V_OFF = kStages * K_BYTES;     // V ring after the K ring
  static constexpr int LDS_BYTES = kStages * (K_BYTES + V_BYTES);
  static constexpr uint32_t TILE_GLOBAL = kBN * D * sizeof(T);  // bytes per tile in HBM
  // loads one wave issues per issue_unit (wave 0 / the others)
  static constexpr int UNIT0 = K_PER_WAVE + V_PER_WAVE;
  static constexpr int UNIT = K_PER_WAVE - (K_EXTRA ? 1 : 0) + V_PER_WAVE;
  static_assert(V_INS % kWaves == 0, "V DMA must split evenly");
  static_assert(K_EXTRA <= 1, "at most wave 0 issues an extra K load");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Per-lane byte offset (within the head's K or V slice, tile 0) of the chunk
// that DMA instruction `ins` places in LDS slot ins*64 + lane.
template <typename T, int D>
__device__ __forceinline__ uint32_t dma_src(int ins, int lane, int stride) {
  const int p = ins * kWave + lane;
  const int row = p / stride;
  const int col = p % stride;
  return col < D / 8 ? (uint32_t)(row * D + col * 8) * sizeof(T) : kOutOfRange;
}

// gfx9 buffer resource (raw, stride 0): base, num_records = bytes, word 3
// as for make_rsrc.  Built by hand so it can be an SGPR operand of asm.
__device__ __forceinline__ u32x4 raw_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, (uint32_t)kRsrcWord3};
}

// One 16-byte-per-lane global -> LDS load (buffer_load_dwordx4 ... lds).  The
// 64 lanes' data land at lds_addr + 16 * lane.  Written as asm so that the
// compiler does not order LDS reads of other ring stages behind it (it
// cannot tell the stages apart and would wait for every load in flight);
// ring_barrier() waits for these loads explicitly.
__device__ __forceinline__ void dma16(u32x4 rs, uint32_t lds_addr, uint32_t voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs),
               "{m0}"(lds_addr)
               : "memory");
}

template <typename T, typename OT, int D, bool CAUSAL>
struct Pipe {
  typedef typename Mfma16<T>::frag frag;
  typedef PipeLayout<T, D> L;
  static constexpr int QF = D / 16;    // K.Q^T MFMAs per 32-key block
  static constexpr int NDB = D / 32;
  static constexpr int NPV = 2 * NDB;  // P.V MFMAs per 32-key block
  static_assert(QF == NPV, "slots pair one K.Q^T with one P.V MFMA");
  static constexpr int NSLOT = QF + NPV;

  int lane, wave, l32, g, qw, my_q, Nk;
  float c;
  uint32_t kbase, vbase;  // per-lane LDS byte addresses of fragment 0
  frag qf[QF];
  f32x16 acc[NDB];
  f32x16 S0, S1;      // S^T blocks (alternate between the two blocks of a tile)
  frag P0[2], P1[2];  // P blocks rounded to T (alternate likewise)
  float m_use;
  float l;   // half-wave sum of p (fp32): gives L
  float lr;  // half-wave sum of p as rounded to T for P.V: normalises O

  __device__ __forceinline__ frag kfrag(const lds_char *kp, int f) const {
    return *(const __attribute__((address_space(3))) frag *)(kp + f * 32);
  }
  __device__ __forceinline__ frag vfrag(const lds_char *vp, int m) const {
    const int ks = m / NDB, db = m % NDB;
    const lds_char *a0 = vp + ks * 16 * L::SV * 16 + db * 64;
    const u32x2 lo = read_tr16(a0);
    const u32x2 hi = read_tr16(a0 + 8 * L::SV * 16);
    const u32x4 raw = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(frag, raw);
  }
  __device__ __forceinline__ const lds_char *kptr(const lds_char *ring, int st,
                                                  int half) const {
    return ring + kbase + st * L::K_BYTES + half * 32 * L::SK * 16;
  }
  __device__ __forceinline__ const lds_char *vptr(const lds_char *ring, int st,
                                                  int half) const {
    return ring + vbase + st * L::V_BYTES + half * 32 * L::SV * 16;
  }

  // S^T of a 32-key block = K Q^T (no overlap; prologue only).
  __device__ __forceinline__ void qk(const lds_char *kp, f32x16 &sc) const {
    sc = f32x16{};
#pragma unroll
    for (int f = 0; f < QF; ++f) sc = Mfma16<T>::mma(kfrag(kp, f), qf[f], sc);
  }

  // acc += V^T P^T of a 32-key block (no overlap; drain only).
  __device__ __forceinline__ void pv(const lds_char *vp, const frag (&pin)[2]) {
#pragma unroll
    for (int m = 0; m < NPV; ++m)
      acc[m % NDB] = Mfma16<T>::mma(vfrag(vp, m), pin[m / NDB], acc[m % NDB]);
  }

  // Hides keys >= Nk and (causal) keys after the row's query: S := -inf.
  __device__ __forceinline__ void mask(f32x16 &sc, int k0) const {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + acc_row(r, g);
      const bool hidden = (key >= Nk) || (CAUSAL && key > my_q);
      sc[r] = hidden ? -INFINITY : sc[r];
    }
  }

  // One 32-key block, software-pipelined by hand.  The MFMA stream
  // alternates K.Q^T of the next block (into sout) with P.V of the previous
  // block (with pin); after each MFMA the wave issues the LDS reads two
  // MFMA pairs ahead and one slice of the softmax of this block (on sin,
  // into pout), so the VALU work runs while the MFMA pipe is busy.  Slices:
  //   0-1   row maximum of the block
  //   2     half-wave exchange, lazy move of the exponent reference, alpha
  //   3-10  p = 2^(c*s - m) and its fp32 sum, two elements per slice
  //   11-12 rounding of p to T (the P.V operand) and the sum of the rounded p
  //   13    l, lr
  // The reference moves per lane, only when the block's maximum exceeds it
  // by more than kLazy (both half-waves of a query take the same decision);
  // acc is then scaled by alpha after the block (a rare, wave-uniform
  // branch).  O is normalised by lr, the sum of p exactly as rounded for
  // P.V, so the weights applied to V sum to one; L uses l.  MASKED: s may
  // hold -inf, and the exponent is clamped so a hidden key gives p = 0 even
  // when c == 0 (where -inf * c is NaN).
  template <bool MASKED>
  __device__ __forceinline__ void block_step(const lds_char *kp, const lds_char *vp,
                                             f32x16 &sin, f32x16 &sout,
                                             const frag (&pin)[2], frag (&pout)[2]) {
    constexpr int NCHUNK = 14;
    frag kf[QF], vf[NPV];
    float mx = 0.f, nm = 0.f, alpha = 1.f, psum = 0.f, rsum = 0.f;
    bool need = false;
    f32x16 pf;  // p in fp32
    sout = f32x16{};

    auto chunk = [&](int ch) {
      // Each slice ends with an empty asm that uses its results: the values
      // must exist at that point, so the compiler cannot sink the slice out
      // of its MFMA slot (e.g. past the rescale branch, towards its use).
      if (ch == 0) {
        mx = fmaxf(sin[0], sin[1]);
#pragma unroll
        for (int r = 2; r < 8; ++r) mx = fmaxf(mx, sin[r]);
        asm volatile("" ::"v"(mx));
      } else if (ch == 1) {
#pragma unroll
        for (int r = 8; r < 16; ++r) mx = fmaxf(mx, sin[r]);
        asm volatile("" ::"v"(mx));
      } else if (ch == 2) {
        const u32x2 sw = __builtin_amdgcn_permlane32_swap(
            __builtin_bit_cast(uint32_t, mx), __builtin_bit_cast(uint32_t, mx), false, false);
        mx = fmaxf(__builtin_bit_cast(float, sw[0]), __builtin_bit_cast(float, sw[1]));
        const float mt = mx * c;  // -inf or NaN when the row sees no key of this block
        need = mt > m_use + kLazy;
        const float m_new = need ? mt : m_use;
        alpha = __builtin_amdgcn_exp2f(m_use - m_new);
        m_use = m_new;
        nm = -m_new;
        asm volatile("" ::"v"(alpha), "v"(nm));
      } else if (ch <= 10) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int r = 2 * (ch - 3) + t;
          float e = __builtin_fmaf(sin[r], c, nm);
          if (MASKED) e = fmaxf(e, -3.0e38f);  // NaN or -inf -> 2^-3e38 = 0
          pf[r] = __builtin_amdgcn_exp2f(e);
          psum += pf[r];
        }
        asm volatile("" ::"v"(pf[2 * (ch - 3)]), "v"(pf[2 * (ch - 3) + 1]), "v"(psum));
      } else if (ch <= 12) {
        const int hh = ch - 11;
        const f32x8 p8 = {pf[8 * hh + 0], pf[8 * hh + 1], pf[8 * hh + 2], pf[8 * hh + 3],
                          pf[8 * hh + 4], pf[8 * hh + 5], pf[8 * hh + 6], pf[8 * hh + 7]};
        pout[hh] = __builtin_convertvector(p8, frag);
        const u32x4 packed = __builtin_bit_cast(u32x4, pout[hh]);
#pragma unroll
        for (int i = 0; i < 4; ++i) rsum = Mfma16<T>::pair_sum(packed[i], rsum);
        asm volatile("" ::"v"(pout[hh]), "v"(rsum));
      } else {
        l = l * alpha + psum;
        lr = lr * alpha + rsum;
        asm volatile("" ::"v"(l), "v"(lr));
      }
    };

    // fragments for the first two MFMA pairs
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      kf[i] = kfrag(kp, i);
      vf[i] = vfrag(vp, i);
    }
#pragma unroll
    for (int i = 0; i < QF; ++i) {
      // K.Q^T, then a slice of the softmax
      sout = Mfma16<T>::mma(kf[i], qf[i], sout);
      if (i + 2 < QF) kf[i + 2] = kfrag(kp, i + 2);
#pragma unroll
      for (int ch = (2 * i) * NCHUNK / NSLOT; ch < (2 * i + 1) * NCHUNK / NSLOT; ++ch)
        chunk(ch);
      __builtin_amdgcn_sched_barrier(0);
      // P.V, then a slice of the softmax
      acc[i % NDB] = Mfma16<T>::mma(vf[i], pin[i / NDB], acc[i % NDB]);
      if (i + 2 < NPV) vf[i + 2] = vfrag(vp, i + 2);
#pragma unroll
      for (int ch = (2 * i + 1) * NCHUNK / NSLOT; ch < (2 * i + 2) * NCHUNK / NSLOT; ++ch)
        chunk(ch);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    }
  }

  // Block b of this wave (its tile-local half and ring stages given): full
  // step, masked step (causal diagonal / key tail), the drain (P.V of the
  // wave's last block) or nothing.
  template <bool ODD>
  __device__ __forceinline__ void block(const lds_char *ring, int b, int lastb,
                                        int vst, int vhalf, int kst, int khalf) {
    f32x16 &sin = ODD ? S1 : S0;
    f32x16 &sout = ODD ? S0 : S1;
    frag(&pin)[2] = ODD ? P0 : P1;
    frag(&pout)[2] = ODD ? P1 : P0;
    const lds_char *kp = kptr(ring, kst, khalf);
    const lds_char *vp = vptr(ring, vst, vhalf);
    if (b <= lastb) {
      const int k0 = b * 32;
      const bool need_mask = (k0 + 32 > Nk) || (CAUSAL && k0 + 31 > qw);
      if (need_mask) {
        mask(sin, k0);
        block_step<true>(kp, vp, sin, sout, pin, pout);
      } else {
        block_step<false>(kp, vp, sin, sout, pin, pout);
      }
    } else if (b == lastb + 1) {
      pv(vp, pin);
    }
  }
};

// Issues the DMA of one K tile and one V tile into their ring stages.
template <typename L>
__device__ __forceinline__ void issue_unit(u32x4 k_rs, u32x4 v_rs, uint32_t ring_addr,
                                           const uint32_t *ksrc, const uint32_t *vsrc,
                                           int wave, int ktile, int vtile) {
  const uint32_t koff = (uint32_t)ktile * L::TILE_GLOBAL;
  const uint32_t voff = (uint32_t)vtile * L::TILE_GLOBAL;
  const uint32_t kst = ktile & (kStages - 1), vst = vtile & (kStages - 1);
#pragma unroll
  for (int i = 0; i < L::K_PER_WAVE; ++i) {
    if (i < L::K_PER_WAVE - 1 || L::K_EXTRA == 0 || wave < L::K_EXTRA) {
      const uint32_t ins = i * kWaves + wave;
      dma16(k_rs, ring_addr + kst * L::K_BYTES + ins * kWave * 16, ksrc[i] + koff);
    }
  }
#pragma unroll
  for (int i = 0; i < L::V_PER_WAVE; ++i) {
    const uint32_t ins = i * kWaves + wave;
    dma16(v_rs, ring_addr + L::V_OFF + vst * L::V_BYTES + ins * kWave * 16, vsrc[i] + voff);
  }
}

template <typename T, typename OT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fa_fwd_pipe(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    OT *__restrict__ o, float *__restrict__ lse, int Nq, int Nk, int BH, int nqt,
    float c, int negate) {
  typedef Pipe<T, OT, D, CAUSAL> P;
  typedef typename P::L L;
  typedef typename P::frag frag;
  __shared__ __attribute__((aligned(16))) char ring_[L::LDS_BYTES];
  lds_char *ring = (lds_char *)ring_;
  const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;

  P s;
  const int tid = threadIdx.x;
  s.lane = tid & 63;
  // wave-uniform: keeps the per-wave causal decisions in scalar branches
  s.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  s.l32 = s.lane & 31;
  s.g = s.lane >> 5;
  s.Nk = Nk;
  s.c = c;
  s.kbase = (uint32_t)(s.l32 * L::SK + s.g) * 16;
  {
    const int G = s.lane >> 4, s16 = s.lane & 15;
    const int row = 4 * (G >> 1) + (s16 >> 2);
    const int col = 16 * (G & 1) + 4 * (s16 & 3);  // element within the 32-wide d block
    s.vbase = (uint32_t)L::V_OFF + (uint32_t)row * L::SV * 16 + (uint32_t)col * 2;
  }

  const WorkItem wi = work_item(BH, nqt, CAUSAL);
  s.qw = wi.q0 + s.wave * 32;
  s.my_q = s.qw + s.l32;
  const size_t qoff = (size_t)wi.bh * Nq * D;
  const size_t koff = (size_t)wi.bh * Nk * D;
  const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(q + qoff, (uint32_t)Nq * D * sizeof(T));
  const u32x4 k_rs = raw_rsrc(k + koff, (uint32_t)Nk * D * sizeof(T));
  const u32x4 v_rs = raw_rsrc(v + koff, (uint32_t)Nk * D * sizeof(T));

  uint32_t ksrc[L::K_PER_WAVE], vsrc[L::V_PER_WAVE];
#pragma unroll
  for (int i = 0; i < L::K_PER_WAVE; ++i)
    ksrc[i] = dma_src<T, D>(i * kWaves + s.wave, s.lane, L::SK);
#pragma unroll
  for (int i = 0; i < L::V_PER_WAVE; ++i)
    vsrc[i] = dma_src<T, D>(i * kWaves + s.wave, s.lane, L::SV);

  const int kend = CAUSAL ? min(Nk, wi.q0 + kBM) : Nk;
  const int nkt = (kend + kBN - 1) / kBN;
  // last 32-key block this wave needs
  const int lastb = CAUSAL ? min(2 * nkt - 1, s.qw / 32) : 2 * nkt - 1;

  // Rows past Nk may be left unwritten by the bounds-checked loads; start
  // the ring at zero so such rows hold finite values.
  for (int i = tid; i < L::LDS_BYTES / 16; i += kThreads)
    *(__attribute__((address_space(3))) u32x4 *)(ring + i * 16) = u32x4{};
  __syncthreads();

#pragma unroll
  for (int f = 0; f < P::QF; ++f) {
    const uint32_t off = ((uint32_t)s.my_q * D + 16 * f + 8 * s.g) * sizeof(T);
    u32x4 raw = load16(q_rs, off);
    if (negate) raw ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    s.qf[f] = __builtin_bit_cast(frag, raw);
  }
  // Q must be in registers before the ring's loads are counted by vmcnt.
  wait_vmcnt<0>();
  // Prologue units: (K0,V0) (K1,V1) (K2,V2).  Step j then issues (K(j+3),
  // V(j+2)); every unit has the same per-wave load count, so "the previous
  // unit may still be in flight" is one vmcnt value.
  issue_unit<L>(k_rs, v_rs, ring_addr, ksrc, vsrc, s.wave, 0, 0);
  issue_unit<L>(k_rs, v_rs, ring_addr, ksrc, vsrc, s.wave, 1, 1);
  issue_unit<L>(k_rs, v_rs, ring_addr, ksrc, vsrc, s.wave, 2, 2);
  if (L::K_EXTRA && s.wave < L::K_EXTRA)
    ring_barrier<2 * L::UNIT0>();  // (K0,V0) landed
  else
    ring_barrier<2 * L::UNIT>();

#pragma unroll
  for (int db = 0; db < P::NDB; ++db) s.acc[db] = f32x16{};
  s.m_use = -INFINITY;
  s.l = 0.f;
  s.lr = 0.f;
  s.P1[0] = frag{};  // P.V of block -1 adds nothing
  s.P1[1] = frag{};
  s.qk(s.kptr(ring, 0, 0), s.S0);

  // Tile step j reads K tiles j, j+1 and V tiles j-1, j:
  //   block 2j  : P.V(V tile j-1, rows 32..63), K.Q^T(K tile j, rows 32..63)
  //   block 2j+1: P.V(V tile j, rows 0..31),    K.Q^T(K tile j+1, rows 0..31)
  // K(j+1) and V(j) were requested two steps earlier; the unit requested in
  // step j-1 may still be in flight.  Step j requests K(j+3) into the stage
  // of K(j-1) and V(j+2) into the stage of V(j-2), both last read in step
  // j-1.  Every wave runs every step so that the loads and barriers line up.
  const int nsteps = nkt + 1;
  for (int j = 0; j < nsteps; ++j) {
    if (L::K_EXTRA && s.wave < L::K_EXTRA)
      ring_barrier<L::UNIT0>();
    else
      ring_barrier<L::UNIT>();
    issue_unit<L>(k_rs, v_rs, ring_addr, ksrc, vsrc, s.wave, j + 3, j + 2);
    const int st0 = j & (kStages - 1);
    const int stm = (j + kStages - 1) & (kStages - 1);
    const int st1 = (j + 1) & (kStages - 1);
    s.template block<false>(ring, 2 * j, lastb, stm, 1, st0, 1);
    s.template block<true>(ring, 2 * j + 1, lastb, st0, 0, st1, 0);
  }
  wait_vmcnt<0>();  // no DMA may outlive the workgroup's LDS

  epilogue<D, OT>(s.acc, s.m_use, s.l, o, lse, wi.bh, Nq, s.my_q, s.g, s.lr);
}

// ---------------------------------------------------------------------------
// fp32 inputs: same structure on v_mfma_f32_32x32x2_f32 (true fp32 products).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fa_fwd_f32(
    const float *__restrict__ q, const float *__restrict__ k,
    const float *__restrict__ v, float *__restrict__ o, float *__restrict__ lse,
    int Nq, int Nk, int BH, int nqt, float c) {
  constexpr int KS = D + 1;            // K row stride (floats): 32 rows on 32 banks
  constexpr int VS = D;                // V row stride (floats)
  constexpr int K_ELEMS = kBN * KS;
  constexpr int BUF = K_ELEMS + kBN * VS;
  constexpr int CPR = D / 4;           // 16-byte chunks per row
  constexpr int NCH = kBN * CPR;
  constexpr int LPT = (NCH + kThreads - 1) / kThreads;
  constexpr int HD = D / 2;            // head-dim entries per half-wave
  constexpr int NDB = (D < 32 ? 32 : D) / 32;

  __shared__ __attribute__((aligned(16))) float smem[2 * BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const WorkItem wi = work_item(BH, nqt, CAUSAL);
  const int qw = wi.q0 + wave * 32;
  const int my_q = qw + l32;

  const size_t qoff = (size_t)wi.bh * Nq * D;
  const size_t koff = (size_t)wi.bh * Nk * D;
  const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(q + qoff, (uint32_t)Nq * D * 4u);
  const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(k + koff, (uint32_t)Nk * D * 4u);
  const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(v + koff, (uint32_t)Nk * D * 4u);

  // The MFMA k index of half-wave g at step t stands for head-dim entry
  // g*D/2 + t, for Q and K alike, so each lane loads a contiguous half row.
  float qf[HD];
#pragma unroll
  for (int f = 0; f < HD / 4; ++f) {
    const uint32_t off = ((uint32_t)my_q * D + g * HD + 4 * f) * 4u;
    const f32x4 x = __builtin_bit_cast(f32x4, load16(q_rs, off));
    qf[4 * f + 0] = x[0];
    qf[4 * f + 1] = x[1];
    qf[4 * f + 2] = x[2];
    qf[4 * f + 3] = x[3];
  }

  u32x4 kreg[LPT], vreg[LPT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int ch = tid + i * kThreads;
      if (NCH % kThreads == 0 || ch < NCH) {
        const int row = ch / CPR;
        const int col = (ch % CPR) * 4;
        const uint32_t off = ((uint32_t)(kt * kBN + row) * D + col) * 4u;
        kreg[i] = load16(k_rs, off);
        vreg[i] = load16(v_rs, off);
      }
    }
  };
  auto swrite = [&](int buf) {
    float *Ks = smem + buf * BUF;
    float *Vs = Ks + K_ELEMS;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int ch = tid + i * kThreads;
      if (NCH % kThreads == 0 || ch < NCH) {
        const int row = ch / CPR;
        const int col = (ch % CPR) * 4;
        const f32x4 kx = __builtin_bit_cast(f32x4, kreg[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) Ks[row * KS + col + e] = kx[e];
        *reinterpret_cast<u32x4 *>(Vs + row * VS + col) = vreg[i];
      }
    }
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  const int kend = CAUSAL ? min(Nk, wi.q0 + kBM) : Nk;
  const int nkt = (kend + kBN - 1) / kBN;

  gload(0);
  swrite(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) gload(kt + 1);
    const int k0 = kt * kBN;
    const bool active = !CAUSAL || (k0 <= qw + 31);
    if (active) {
      const float *Ks = smem + (kt & 1) * BUF;
      const float *Vs = Ks + K_ELEMS;
      f32x16 s[kBN / 32];
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb) {
        s[kb] = f32x16{};
        const float *krow = Ks + (kb * 32 + l32) * KS + g * HD;
#pragma unroll
        for (int t = 0; t < HD; ++t)
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[t], qf[t], s[kb], 0, 0, 0);
      }
      const bool need_mask = (k0 + kBN > Nk) || (CAUSAL && k0 + kBN - 1 > qw);
      scale_and_mask<CAUSAL>(s, c, k0, Nk, my_q, g, need_mask);
      const float alpha = online_softmax(s, m, l);
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + acc_row(r, g);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int d = db * 32 + l32;
            const float a = (D >= 32 || d < D) ? Vs[key * VS + (d < D ? d : 0)] : 0.f;
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[kb][r], acc[db], 0, 0, 0);
          }
        }
      }
    }
    if (kt + 1 < nkt) swrite((kt + 1) & 1);
    __syncthreads();
  }

  epilogue<D, float>(acc, m, l, o, lse, wi.bh, Nq, my_q, g);
}

// ---------------------------------------------------------------------------
// Host side.

thread_local char g_hip_error[256] = "";

int hip_fail(hipError_t e) {
  snprintf(g_hip_error, sizeof(g_hip_error), "%s: %s", hipGetErrorName(e),
           hipGetErrorString(e));
  return FA_ERR_HIP;
}

struct Launch {
  const void *q, *k, *v;
  void *o;
  float *lse;
  int Nq, Nk, BH, nqt;
  float c;
  hipStream_t stream;
};

template <typename T, typename OT, int D, bool CAUSAL>
hipError_t launch16(const Launch &a) {
  const dim3 grid((unsigned)(a.BH * a.nqt)), block(kThreads);
  if constexpr (D >= 64) {
    // c >= 0 here; a negative scale flips the sign of Q inside the kernel.
    const float c = a.c < 0.f ? -a.c : a.c;
    hipLaunchKernelGGL((fa_fwd_pipe<T, OT, D, CAUSAL>), grid, block, 0, a.stream,
                       (const T *)a.q, (const T *)a.k, (const T *)a.v, (OT *)a.o, a.lse,
                       a.Nq, a.Nk, a.BH, a.nqt, c, a.c < 0.f ? 1 : 0);
  } else {
    hipLaunchKernelGGL((fa_fwd_mfma16<T, OT, D, CAUSAL>), grid, block, 0, a.stream,
                       (const T *)a.q, (const T *)a.k, (const T *)a.v, (OT *)a.o, a.lse,
                       a.Nq, a.Nk, a.BH, a.nqt, a.c);
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch32(const Launch &a) {
  const dim3 grid((unsigned)(a.BH * a.nqt)), block(kThreads);
  hipLaunchKernelGGL((fa_fwd_f32<D, CAUSAL>), grid, block, 0, a.stream,
                     (const float *)a.q, (const float *)a.k, (const float *)a.v,
                     (float *)a.o, a.lse, a.Nq, a.Nk, a.BH, a.nqt, a.c);
  return hipGetLastError();
}

template <typename T, typename OT, int D>
hipError_t dispatch16_causal(const Launch &a, bool causal) {
  return causal ? launch16<T, OT, D, true>(a) : launch16<T, OT, D, false>(a);
}

template <typename T, typename OT>
hipError_t dispatch16(const Launch &a, int D, bool causal) {
  switch (D) {
    case 16: return dispatch16_causal<T, OT, 16>(a, causal);
    case 32: return dispatch16_causal<T, OT, 32>(a, causal);
    case 64: return dispatch16_causal<T, OT, 64>(a, causal);
    default: return dispatch16_causal<T, OT, 128>(a, causal);
  }
}

hipError_t dispatch32(const Launch &a, int D, bool causal) {
  switch (D) {
    case 16: return causal ? launch32<16, true>(a) : launch32<16, false>(a);
    case 32: return causal ? launch32<32, true>(a) : launch32<32, false>(a);
    case 64: return causal ? launch32<64, true>(a) : launch32<64, false>(a);
    default: return causal ? launch32<128, true>(a) : launch32<128, false>(a);
  }
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

int fa_version(void) { return 100; }

const char *fa_status_str(int s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULLPTR: return "null pointer argument";
    case FA_ERR_SHAPE: return "invalid shape (B, H, Nq, Nk must be >= 1 and sizes must fit)";
    case FA_ERR_HEAD_DIM: return "unsupported head dimension (D must be 16, 32, 64 or 128)";
    case FA_ERR_DTYPE: return "unknown dtype";
    case FA_ERR_SCALE: return "scale is not finite";
    case FA_ERR_ALIGN: return "misaligned pointer (q, k, v, o need 16 bytes, lse 4)";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_OVERLAP: return "output buffers overlap the inputs";
    default: return "unknown status";
  }
}

const char *fa_last_hip_error(void) { return g_hip_error; }

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
           int64_t H, int64_t Nq, int64_t Nk, int64_t D, float scale, int causal,
           int dtype, void *stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULLPTR;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  if (D != 16 && D != 32 && D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  if (dtype < FA_F32 || dtype > FA_F16_OF32) return FA_ERR_DTYPE;
  if (!isfinite(scale)) return FA_ERR_SCALE;

  const int64_t in_size = (dtype == FA_F32) ? 4 : 2;
  const int64_t out_size = (dtype == FA_F32 || dtype == FA_BF16_OF32 || dtype == FA_F16_OF32) ? 4 : 2;
  // Per-head slices are addressed with 32-bit byte offsets (plus one tile of
  // slack past the end for ragged rows); the grid is one-dimensional.
  const int64_t lim = (int64_t)1 << 31;
  if (Nq > lim / (D * 4) - kBM || Nk > lim / (D * 4) - kBN) return FA_ERR_SHAPE;
  const int64_t BH = B * H;
  if (B > lim || H > lim || BH > lim) return FA_ERR_SHAPE;
  const int64_t nqt = (Nq + kBM - 1) / kBM;
  if (BH * nqt >= lim) return FA_ERR_SHAPE;

  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGN;
  if ((uintptr_t)lse & 3u) return FA_ERR_ALIGN;

  const size_t qb = (size_t)(BH * Nq * D * in_size), kb = (size_t)(BH * Nk * D * in_size);
  const size_t ob = (size_t)(BH * Nq * D * out_size), lb = (size_t)(BH * Nq * 4);
  if (overlaps(o, ob, q, qb) || overlaps(o, ob, k, kb) || overlaps(o, ob, v, kb) ||
      overlaps(lse, lb, q, qb) || overlaps(lse, lb, k, kb) || overlaps(lse, lb, v, kb) ||
      overlaps(o, ob, lse, lb))
    return FA_ERR_OVERLAP;

  Launch a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.Nq = (int)Nq;
  a.Nk = (int)Nk;
  a.BH = (int)BH;
  a.nqt = (int)nqt;
  a.c = scale * 1.4426950408889634f;
  a.stream = (hipStream_t)stream;

  hipError_t e;
  const bool cz = causal != 0;
  switch (dtype) {
    case FA_F32: e = dispatch32(a, (int)D, cz); break;
    case FA_BF16: e = dispatch16<__bf16, __bf16>(a, (int)D, cz); break;
    case FA_BF16_OF32: e = dispatch16<__bf16, float>(a, (int)D, cz); break;
    case FA_F16: e = dispatch16<_Float16, _Float16>(a, (int)D, cz); break;
    default: e = dispatch16<_Float16, float>(a, (int)D, cz); break;
  }
  if (e != hipSuccess) return hip_fail(e);
  return FA_OK;
}

}  // extern "C"
