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
// gfx950 mapping (16-bit inputs; fp32 inputs use fa_fwd_f32 further down):
//   * Workgroups of eight wave64s, two per SIMD, each wave holding 32 query
//     rows: 256 rows per workgroup, or 128 with the two waves of a SIMD
//     splitting the key blocks of the same rows (pair-split layout, when
//     query tiles are few); see pipe8_run.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_{bf16,f16} puts one query per lane
//     column: lane l owns query (l mod 32) and 16 of each 32-key block, so a
//     row maximum or sum is a reduction inside the lane plus one exchange with
//     lane l^32.  The S^T accumulator registers, rounded to the input type,
//     are exactly the B operand of O^T += V^T P^T: no trip of P through LDS.
//   * K and V tiles of 64 keys go global -> LDS directly (buffer_load ...
//     lds) into four-stage rings, one barrier per tile; K rows are read with
//     ds_read_b128, V^T fragments with ds_read_b64_tr_b16; row strides are
//     padded so that neither read has bank conflicts.
//   * Ragged tails: every global read goes through a buffer resource whose
//     size is the (batch, head) slice, so rows past Nq / Nk read as zero;
//     scores of keys >= Nk are -inf, rows >= Nq are never stored.
//   * Causal: blocks past a wave's last query are never visited; only the
//     diagonal block (and a key tail) is masked.
//   * Work distribution: fa_fwd runs one workgroup per query tile, longest
//     causal tiles first; fa_fwd_ws runs a stream-K schedule (equal shares
//     of (query tile, key tile) units per compute unit, cut tiles combined
//     by fa_merge_stream) when query tiles are too few to balance.
//   * The softmax works in base 2: c = scale*log2(e) is folded into the
//     scores, p = 2^(c*s - m2), and L = ln2 * (m2 + log2 l).

#include <hip/hip_runtime.h>
#include <type_traits>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "fa.h"
#include "mask.h"
#include "mma16.h"
#include "stream_plan.h"

namespace {

using namespace fa_sched;

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per tile

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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

__device__ __forceinline__ WorkItem work_item(int BH, int nqt, bool causal, int rows = kBM) {
  const int id = blockIdx.x;
  const int bh = id % BH;
  const int t = id / BH;
  const int qt = causal ? (nqt - 1 - t) : t;
  return {bh, qt * rows};
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
  // a row that has seen no visible key yet (possible when the keys are
  // split, a chunk starting past the row) keeps p = 0 and alpha = 0
  const float mu = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m - mu);
  float psum = 0.f;
#pragma unroll
  for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(s[kb][r] - mu);
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

// Writes O = acc / lo (rows < Nq) and L = ln2 * (m + log2 l).  l is a
// half-wave partial sum; lo, the normaliser of O, is the row's whole sum (by
// default l itself, both halves added).
// Four values in a storage type, as the raw register words a store takes.
template <typename OT> struct Pack4;
template <> struct Pack4<float> {
  typedef u32x4 type;
  static __device__ __forceinline__ type pack(f32x4 v) { return __builtin_bit_cast(u32x4, v); }
};
template <> struct Pack4<__bf16> {
  typedef u32x2 type;
  static __device__ __forceinline__ type pack(f32x4 v) {
    return __builtin_bit_cast(u32x2, __builtin_convertvector(v, bf16x4));
  }
};
template <> struct Pack4<_Float16> {
  typedef u32x2 type;
  static __device__ __forceinline__ type pack(f32x4 v) {
    return __builtin_bit_cast(u32x2, __builtin_convertvector(v, f16x4));
  }
};

// Stores a lane's row values (acc * inv) from registers that nothing
// overwrites afterwards: every value is computed before the first store.
// Computing each store's data into the same few registers made each one
// wait until the previous store had read its data, which under load from
// other waves serialised the stores.
// Column blocks [cb, ce) of the row (wave-uniform bounds).
template <typename OT, int NDB>
__device__ __forceinline__ void store_row(const f32x16 (&acc)[NDB], float inv, OT *orow, int g,
                                          int dlim, int cb = 0, int ce = NDB) {
  typedef typename Pack4<OT>::type PT;
  PT pk[NDB * 4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 v = {acc[db][4 * r4 + 0] * inv, acc[db][4 * r4 + 1] * inv,
                       acc[db][4 * r4 + 2] * inv, acc[db][4 * r4 + 3] * inv};
      pk[db * 4 + r4] = Pack4<OT>::pack(v);
    }
#pragma unroll
  for (int i = 0; i < NDB * 4; ++i) asm volatile("" : "+v"(pk[i]));
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = db * 32 + 8 * r4 + 4 * g;
      if (db >= cb && db < ce && d < dlim) *reinterpret_cast<PT *>(orow + d) = pk[db * 4 + r4];
    }
}

template <int D, typename OT>
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[(D < 32 ? 32 : D) / 32],
                                         float m, float l, OT *o, float *lse, int bh,
                                         int Nq, int my_q, int g, float lo = -1.f,
                                         float osc = 1.f, int cb = 0,
                                         int ce = (D < 32 ? 32 : D) / 32, bool stats = true) {
  const float lt = l + __shfl_xor(l, 32);
  const float lot = lo < 0.f ? lt : lo;
  if (my_q >= Nq) return;
  // a row that saw no key (possible under the window mask) stores O = 0;
  // osc: a factor of O (1 except on the FP8 path)
  const float inv = (lot > 0.f ? 1.0f / lot : 0.f) * osc;
  OT *orow = o + ((size_t)bh * Nq + my_q) * D;
  store_row<OT, (D < 32 ? 32 : D) / 32>(acc, inv, orow, g, D, cb, ce);
  if (stats && g == 0) lse[(size_t)bh * Nq + my_q] = (m + log2f(lt)) * 0.69314718055994531f;
}

// ---------------------------------------------------------------------------
// Pipelined kernel for 16-bit inputs (D = 16, 32, 64, 128).
//
//   * Products are transposed: S^T = K.Q^T on v_mfma_f32_32x32x16 (bf16 or
//     fp16, fp32 accumulation) puts one query per lane (lane l holds query
//     l % 32, 16 of its 32 scores per block, half-wave l / 32 the other
//     rows), so row reductions are in-lane plus one exchange; P^T, rounded
//     to the input type, is the B operand of O^T = V^T.P^T directly, with no
//     trip through LDS.
//   * K and V tiles (64 keys) go global -> LDS directly (buffer_load ... lds,
//     16 bytes per lane, written lane-linearly) into a K ring and a V ring of
//     four stages each; nothing passes through VGPRs.  Tile t+3 of K and
//     tile t+2 of V are requested while tile t is computed on.
//   * Rows are padded in LDS (PipeLayout): K rows so that the 16 rows read by
//     one ds_read_b128 pass start on distinct bank groups; V rows where the
//     transpose reads below are fastest.  Padding slots are loaded from an out-of-range offset (zero, no
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
//   * No row maximum per block: each block is exponentiated against the
//     current reference, and the reference moves (to the exact maximum, with
//     the accumulator rescaled) only when a lane's p of the block sum past
//     2^kLazy, or on a wave's first block; the check is one compare and a
//     wave-uniform branch.  p stays at most 2^kLazy and O = acc / l is
//     unchanged (the update rule of the online softmax with a reference that
//     lags the maximum; the rescaling is exact).
//   * Half-wave maxima (on a move) are exchanged with v_permlane32_swap.
//   * A negative scale is applied by flipping the sign bits of the Q
//     fragments once (exact), so the folded factor c is never negative.

constexpr int kLazy = 8;
// A block whose p (16 per lane) sum to more than this moves the reference.
constexpr float kSumMax = (float)(1 << kLazy);
// Two ones of type T packed in a word (the A operand of the rounded-sum MFMA).
template <typename T> __device__ __forceinline__ constexpr uint32_t kOne2();
template <> __device__ __forceinline__ constexpr uint32_t kOne2<__bf16>() { return 0x3f803f80u; }
template <> __device__ __forceinline__ constexpr uint32_t kOne2<_Float16>() { return 0x3c003c00u; }
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

// s_waitcnt vmcnt(N) lgkmcnt(L) (gfx9 encoding; L = 15: no LDS wait).
template <int N, int L = 15>
__device__ __forceinline__ void wait_counts() {
  static_assert(N >= 0 && N < 64 && L >= 0 && L < 16, "counter range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (L << 8));
}

// Debug builds (compiled with -DFA_DEBUG_BARRIERS=1, libfa_debug.so): every
// ring barrier also checks that all waves of the workgroup have passed as
// many ring barriers as this one.  The DMA ring's stage accounting assumes
// that they do; a wave that skipped or added a barrier would otherwise let a
// load overwrite a stage still being read, silently.  Each wave counts its
// barriers in its own LDS slot, raised before the barrier; after it, another
// wave's count may be one ahead (raised for the next barrier, which cannot
// complete without this wave) but never behind or further ahead.  A mismatch
// adds one to a device counter that fa_debug_barrier_faults reads
// (include/fa_debug.h).  Release builds compile none of it.
#ifndef FA_DEBUG_BARRIERS
#define FA_DEBUG_BARRIERS 0
#endif
#if FA_DEBUG_BARRIERS
__device__ unsigned int fa_dbg_faults;
__device__ __forceinline__ __attribute__((address_space(3))) unsigned int *dbg_slots() {
  __shared__ unsigned int slots[16];
  return (__attribute__((address_space(3))) unsigned int *)slots;
}
// at the start of every kernel that uses ring barriers
__device__ __forceinline__ void dbg_begin() {
  if (threadIdx.x < 16) dbg_slots()[threadIdx.x] = 0u;
  __syncthreads();
}
__device__ __forceinline__ void dbg_pre() {
  if ((threadIdx.x & 63) == 0) dbg_slots()[threadIdx.x >> 6] += 1u;
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (0x7 << 4) | (0 << 8));  // lgkmcnt(0)
}
__device__ __forceinline__ void dbg_post() {
  const int lane = threadIdx.x & 63, nw = (int)(blockDim.x >> 6);
  const unsigned int mine = dbg_slots()[threadIdx.x >> 6];
  bool bad = false;
  if (lane < nw) {
    const unsigned int d = dbg_slots()[lane] - mine;
    bad = d > 1u;
  }
  if (__ballot(bad) != 0ull && lane == 0) atomicAdd(&fa_dbg_faults, 1u);
}
#define FA_DBG_BEGIN() dbg_begin()
#else
#define FA_DBG_BEGIN() ((void)0)
#endif
template <int N, bool LGKM0 = false>
__device__ __forceinline__ void wait_vmcnt() {
  wait_counts<N, LGKM0 ? 0 : 15>();
}

// Workgroup barrier for the DMA ring.  Waits until at most N of this wave's
// buffer loads are in flight and all of its LDS reads but the L youngest
// have returned (LDS accesses of a wave complete in order), then meets the
// other waves.  No memory fence: a workgroup fence would wait for every
// load in flight (vmcnt(0)) and drain the ring.  The empty asm statements
// keep the compiler from moving LDS accesses across.
template <int N, int L = 0>
__device__ __forceinline__ void ring_barrier() {
#if FA_DEBUG_BARRIERS
  dbg_pre();
#endif
  wait_counts<N, L>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#if FA_DEBUG_BARRIERS
  dbg_post();
#endif
}

// ring_barrier<2n> for a wave-uniform n in 0..3: n = this wave's own count
// of K-tile loads (waves differ when a tile's instructions do not divide
// evenly over the eight).
__device__ __forceinline__ void ring_barrier_k2(int n) {
  switch (n) {
    case 0: ring_barrier<0>(); break;
    case 1: ring_barrier<2>(); break;
    case 2: ring_barrier<4>(); break;
    default: ring_barrier<6>(); break;
  }
}

// Ring wait with one per-wave load count for every wave.
template <int N, int L = 0>
__device__ __forceinline__ void ring_barrier_sel(bool one) {
  if (one)
    ring_barrier<N, L>();
  else
    ring_barrier<0, L>();
}

// 16-byte buffer load into registers, as asm: the compiler does not count it
// among the loads it waits for, so its wait must be explicit (loads return
// in issue order, so a later wait that covers younger loads covers it).
__device__ __forceinline__ u32x4 load16_async(u32x4 rs, uint32_t voff) {
  u32x4 r;
  asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(r) : "v"(voff), "s"(rs));
  return r;
}

template <typename T, int D, typename KT = T>
struct PipeLayout {
  static constexpr int C = D / 8;                     // 16-byte chunks per V row
  static constexpr int KRB = D * (int)sizeof(KT);     // bytes of a K row in HBM
  // K and V row strides (16-byte slots): padded against bank conflicts (a K
  // row is its 16-byte chunks plus one, for 16-bit and 8-bit K alike); at
  // D = 16 the V row holds 4 slots so that the P.V fragments' upper 16
  // head-dim columns read the zeroed padding
  static constexpr int SK = KRB / 16 + 1;
  static constexpr int SV = D == 128 ? 20 : (D == 64 ? 12 : (D == 32 ? 6 : 4));
  static constexpr int K_BYTES = kBN * SK * 16;
  static constexpr int V_BYTES = kBN * SV * 16;
  static constexpr int K_INS = kBN * SK / kWave;      // DMA instructions per K tile
  static constexpr int V_INS = kBN * SV / kWave;
  static constexpr int V_OFF = kStages * K_BYTES;     // V ring after the K ring
  static constexpr int LDS_BYTES = kStages * (K_BYTES + V_BYTES);
  static constexpr uint32_t K_TILE_GLOBAL = kBN * KRB;            // bytes per tile in HBM
  static constexpr uint32_t V_TILE_GLOBAL = kBN * D * sizeof(T);
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Per-lane byte offset (within the head's K or V slice, tile 0) of the chunk
// that DMA instruction `ins` places in LDS slot ins*64 + lane.
__device__ __forceinline__ uint32_t dma_src(int ins, int lane, int stride, int row_bytes) {
  const int p = ins * kWave + lane;
  const int row = p / stride;
  const int col = p % stride;
  return col < row_bytes / 16 ? (uint32_t)(row * row_bytes + col * 16) : kOutOfRange;
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

// Key tiles of one query tile under the local-window + global-token mask, as
// a list of two ranges: list entry v < n1 is key tile v (the global tokens'
// tiles), later entries are band tiles b0 + (v - n1).  Without the mask, or
// when the two ranges meet, the list is the identity (n1 = b0).
struct KeyList {
  int n1, b0;
};

// The score product S^T = K Q^T on Q/K elements of type KT: the 16-bit
// MFMA (16 head-dim entries per instruction), or for bytes holding OCP e4m3
// values the scaled FP8 MFMA v_mfma_scale_f32_32x32x64_f8f6f4 with unit
// block scales (E8M0 127 = 2^0; 64 entries per instruction).  KSTEP entries
// per instruction, FB bytes of them per lane: lane l gives row l % 32 and
// the entries [KSTEP/2 (l / 32), +KSTEP/2) of the step, for K (A) and Q
// (B) alike, so the contraction pairs the same head-dim entries whatever
// order the instruction uses within a lane's slots.
typedef int i32x8 __attribute__((ext_vector_type(8)));
template <typename KT> struct QKOp {
  typedef typename Mma<KT>::frag frag;
  static constexpr int KSTEP = 16;
  static constexpr int FB = 16;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return Mma<KT>::mma(a, b, c);
  }
};
template <> struct QKOp<uint8_t> {
  typedef i32x8 frag;
  static constexpr int KSTEP = 64;
  static constexpr int FB = 32;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

template <typename T, typename OT, int D, bool CAUSAL, bool MASKED = false, typename KT = T>
struct Pipe {
  typedef typename Mma<T>::frag frag;            // P.V operands
  typedef QKOp<KT> QK;
  typedef typename QK::frag kfrag_t;             // K.Q^T operands
  typedef PipeLayout<T, D, KT> L;
  static constexpr int QF = D / QK::KSTEP;       // K.Q^T MFMAs per 32-key block
  // O^T blocks of 32 head-dim rows (at D = 16 the upper 16 rows read zero
  // padding of V and are never stored)
  static constexpr int NDB = (D + 31) / 32;
  static constexpr int NPV = 2 * NDB;  // P.V MFMAs per 32-key block
  // MFMA slots of a block: slot i holds K.Q^T i (i < QF) and P.V i (i < NPV)
  static constexpr int NSL = QF > NPV ? QF : NPV;

  int lane, wave, l32, g, qw, my_q, Nk;
  float c;
  Mask mk;     // the window rule (MASKED)
  KeyList kl;  // the item's key tiles (MASKED)
  // Key tile of list entry v, and first key of list block b (32 keys).
  __device__ __forceinline__ int kt_act(int v) const {
    return MASKED ? (v < kl.n1 ? v : kl.b0 + (v - kl.n1)) : v;
  }
  __device__ __forceinline__ int key0(int b) const {
    return MASKED ? kt_act(b >> 1) * kBN + (b & 1) * 32 : b * 32;
  }
  // Does list block b need the per-score mask (some pair hidden, or keys
  // past Nk)?
  __device__ __forceinline__ bool needs_mask(int k0) const {
    if (MASKED) return k0 + 32 > Nk || !mk.all(qw, qw + 31, k0, k0 + 31);
    return (k0 + 32 > Nk) || (CAUSAL && k0 + 31 > qw);
  }
  uint32_t kbase, vbase;  // per-lane LDS byte addresses of fragment 0
  float osc;              // factor of O (the FP8 path's V descale; else 1)
  kfrag_t qf[QF];
  f32x16 acc[NDB];
  f32x16 S0, S1;      // S^T blocks (alternate between the two blocks of a tile)
  frag P0[2], P1[2];  // P blocks rounded to T (alternate likewise)
  // First K and V fragments of the wave's next block, read during the tail
  // of the current one (blocks chained with PRE)
  static constexpr int PFK = QF < 3 ? QF : 3;   // K fragments read ahead
  static constexpr int PFV = NPV < 3 ? NPV : 3;  // V fragments read ahead
  kfrag_t kpre[PFK];
  frag vpre[PFV];
  float m_use;  // exponent reference (base 2), the same in both half-waves
  float nm;     // -m_use, or 0 while m_use = -inf
  float l;   // half-wave sum of p (fp32): gives L
  // Sums of p as rounded to T for P.V (they normalise O).  LRM (D < 128):
  // accumulated by MFMA, lracc += ones . P^T, so every register of every lane
  // holds its query's whole rounded sum (both half-waves' keys); otherwise a
  // v_dot2 per rounded pair into lr, this half-wave's partial sum.  v_dot2
  // runs on the matrix pipe and does not overlap the MFMAs (measured on
  // MI355X: about 8 cycles each); two extra MFMAs per block cost about as
  // much, and measured faster at D = 64, slower at D = 128.
  static constexpr bool LRM = D < 128;
  f32x16 lracc;
  float lr;
  // the row's whole rounded sum
  __device__ __forceinline__ float lr_total() const {
    return LRM ? lracc[0] : lr + __shfl_xor(lr, 32);
  }
  bool fresh;   // no block of the item seen yet (wave-uniform)

  __device__ __forceinline__ kfrag_t kfrag(const lds_char *kp, int f) const {
    return *(const __attribute__((address_space(3))) kfrag_t *)(kp + f * 2 * QK::FB);
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
    for (int f = 0; f < QF; ++f) sc = QK::mma(kfrag(kp, f), qf[f], sc);
  }

  // acc += V^T P^T of a 32-key block, and its rounded sums into lracc (no
  // overlap; drain only).  Fragments are read two MFMAs ahead, as in
  // block_step: this runs inside the ring loop, where the S and P registers
  // of the pipeline are still live.
  __device__ __forceinline__ void pv(const lds_char *vp, const frag (&pin)[2]) {
    frag vf[NPV];
    vf[0] = vfrag(vp, 0);
    vf[1] = vfrag(vp, 1);
#pragma unroll
    for (int m = 0; m < NPV; ++m) {
      acc[m % NDB] = Mma<T>::mma(vf[m], pin[m / NDB], acc[m % NDB]);
      if (m + 2 < NPV) vf[m + 2] = vfrag(vp, m + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (LRM) {
      lr_mma(pin[0]);
      lr_mma(pin[1]);
    }
  }

  // Hides keys >= Nk and (causal) keys after the row's query: S := -inf.
  __device__ __forceinline__ void mask(f32x16 &sc, int k0) const {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + acc_row(r, g);
      const bool hidden =
          MASKED ? (key >= Nk || !mk.visible(my_q, key)) : ((key >= Nk) || (CAUSAL && key > my_q));
      sc[r] = hidden ? -INFINITY : sc[r];
    }
  }

  // The softmax of one block (on s, scaled to base 2 by c) against the
  // current reference nm = -m_use, straight-line: p = 2^(c*s + nm) rounded
  // in pairs into pw, fp32 sum into *ps, rounded sum into *rs (without LRM).
  __device__ __forceinline__ void softmax_block(const f32x16 &s, u32x4 (&pw)[2], float &ps,
                                                float &rs) const {
    float psa = 0.f, psb = 0.f, rsa = 0.f, rsb = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * w], c, nm));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * w + 1], c, nm));
      psa += p0;
      psb += p1;
      const uint32_t wq = Mma<T>::pack2(p0, p1);
      pw[w / 4][w % 4] = wq;
      if (!LRM) {
        if (w & 1)
          rsb = Mma<T>::pair_sum(wq, rsb);
        else
          rsa = Mma<T>::pair_sum(wq, rsa);
      }
    }
    ps = psa + psb;
    rs = rsa + rsb;
  }

  // lracc += ones . P^T for the 16 keys of one P.V operand (rounded sums).
  __device__ __forceinline__ void lr_mma(const frag &p) {
    const frag ones = __builtin_bit_cast(frag, u32x4{kOne2<T>(), kOne2<T>(), kOne2<T>(), kOne2<T>()});
    lracc = Mma<T>::mma(ones, p, lracc);
  }

  // Moves the exponent reference to the exact maximum of block s (and of
  // the blocks before it) and rescales what was accumulated against the old
  // reference: acc, l and lracc by alpha = 2^(m_old - m_new).  Both half-waves
  // of a query take the same maximum (one exchange with lane l ^ 32).  A row
  // that has seen no key keeps m_use = -inf and nm = 0 (hidden scores are
  // -inf, so its p stay 0).
  __device__ __forceinline__ void move_reference(const f32x16 &s) {
    float m3[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) m3[i] = fmaxf(fmaxf(s[3 * i], s[3 * i + 1]), s[3 * i + 2]);
    float mx = fmaxf(fmaxf(fmaxf(m3[0], m3[1]), fmaxf(m3[2], m3[3])), fmaxf(m3[4], s[15]));
    // v_permlane32_swap exchanges the upper half of its first register with
    // the lower half of its second; with both holding mx, each lane finds
    // its partner's maximum in one of the two results.  The results are
    // copied to scalars before the bit casts: __builtin_bit_cast of an
    // element of an ext_vector_type value reads element 0 whatever the index
    // (seen with this compiler), which had reduced the maximum to the lower
    // half's (a row whose keys of the block all sit in the upper half kept
    // its reference at -inf).
    const u32x2 sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mx),
                                                      __builtin_bit_cast(uint32_t, mx), false,
                                                      false);
    const uint32_t sw0 = sw[0], sw1 = sw[1];
    mx = fmaxf(__builtin_bit_cast(float, sw0), __builtin_bit_cast(float, sw1));
    const float m_new = fmaxf(m_use, mx * c);  // -inf while no key is visible
    // exactly 1 when the reference stays (also while it is still -inf)
    const float alpha = m_new > m_use ? __builtin_amdgcn_exp2f(m_use - m_new) : 1.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    l *= alpha;
    if (LRM)
      lracc *= alpha;
    else
      lr *= alpha;
    m_use = m_new;
    nm = m_new == -INFINITY ? 0.f : -m_new;
  }

  // One 32-key block, software-pipelined by hand.  The MFMA stream
  // alternates K.Q^T of the next block (into sout) with P.V of the previous
  // block (with pin); after each MFMA the wave issues the LDS reads three
  // MFMA slots ahead and one slice of the softmax of this block (on sin,
  // into pout), so the VALU work runs while the MFMA pipe is busy.  The
  // slices take the sixteen elements through four stages (exponent, 2^x,
  // fp32 sums and rounding to T into one packed word of the P.V operand,
  // the rounded pair's sum by v_dot2 unless LRM), one pair per slice, each
  // stage one slice behind the previous; the last slice checks the block.
  // With LRM two more MFMAs add the previous block's rounded p to lracc
  // (ones . P^T).
  //
  // The exponent reference is not moved block by block.  Each block is
  // exponentiated against the current reference (p = 2^(c*s - m_use)), and
  // only when some lane's p of the block sum to more than 2^kLazy (so some
  // p may exceed 2^kLazy, or overflowed), or on the wave's first block of an
  // item, does the wave take a rare, wave-uniform path: move the reference
  // to the exact maximum (move_reference, which rescales acc, l and lr) and
  // recompute the block.  So every p that reaches P.V or the sums is at most
  // 2^kLazy, as with a reference that follows the maximum lazily, without a
  // row maximum per block.  O is normalised by lr, the sum of p exactly as
  // rounded for P.V (the weights applied to V sum to one); L uses l.  Hidden
  // keys hold s = -inf and give p = 0 (c > 0 always: the host never passes
  // 0).  One code path serves masked and unmasked blocks, so the
  // accumulators stay in the same registers from block to block.
  // PRE: the first PFK / PFV fragments of this block were read ahead into
  // kpre and vpre, and this block reads those of the next one (kpn, vpn) in
  // its last MFMA slots.
  template <bool PRE = false>
  __device__ __forceinline__ void block_step(const lds_char *kp, const lds_char *vp,
                                             f32x16 &sin, f32x16 &sout,
                                             const frag (&pin)[2], frag (&pout)[2],
                                             const lds_char *kpn = nullptr,
                                             const lds_char *vpn = nullptr) {
    constexpr int NCHUNK = LRM ? 11 : 12;
    kfrag_t kf[QF];
    frag vf[NPV];
    float ea[2], pb[2];        // pair in flight: exponents, then p
    uint32_t wq = 0;           // packed pair waiting for its rounded sum
    float psa = 0.f, psb = 0.f, rsa = 0.f, rsb = 0.f;  // two partial sums each
    bool over = false;
    u32x4 pw[2];  // p rounded to T, packed in pairs (the two P.V operands)
    sout = f32x16{};

    // Softmax slices.  The wave issues in order, so a slice holds only
    // instructions that do not wait on each other.
    auto chunk = [&](int ch) {
      // Each slice ends with an empty asm that uses its results: the values
      // must exist at that point, so the compiler cannot sink the slice out
      // of its MFMA slot (e.g. past the branch, towards its use).
      if (ch < NCHUNK - 1) {
        const int k = ch;  // stage A on pair k, B on k-1, C on k-2, D on k-3
        if (!LRM && k >= 3 && k - 3 < 8) {  // D: sum of the rounded pair
          if ((k - 3) & 1)
            rsb = Mma<T>::pair_sum(wq, rsb);
          else
            rsa = Mma<T>::pair_sum(wq, rsa);
        }
        if (k >= 2 && k - 2 < 8) {  // C: fp32 sums, rounding to T
          const int w = k - 2;
          psa += pb[0];
          psb += pb[1];
          wq = Mma<T>::pack2(pb[0], pb[1]);
          pw[w / 4][w % 4] = wq;
        }
        if (k >= 1 && k - 1 < 8) {  // B: p = 2^x
          pb[0] = __builtin_amdgcn_exp2f(ea[0]);
          pb[1] = __builtin_amdgcn_exp2f(ea[1]);
        }
        if (k < 8) {  // A: exponents of elements 2k, 2k+1
          ea[0] = __builtin_fmaf(sin[2 * k], c, nm);
          ea[1] = __builtin_fmaf(sin[2 * k + 1], c, nm);
        }
        asm volatile("" ::"v"(ea[0]), "v"(ea[1]), "v"(pb[0]), "v"(pb[1]), "v"(wq), "v"(psa),
                     "v"(psb), "v"(rsa), "v"(rsb));
      } else {
        psa += psb;
        rsa += rsb;
        // a NaN sum (never from finite inputs) does not trigger
        over = psa > kSumMax;
        asm volatile("" ::"v"(psa), "v"(rsa));
      }
    };

    // fragments are read up to three MFMA slots ahead
#pragma unroll
    for (int i = 0; i < (PFK > PFV ? PFK : PFV); ++i) {
      if (i < PFK) kf[i] = PRE ? kpre[i] : kfrag(kp, i);
      if (i < PFV) vf[i] = PRE ? vpre[i] : vfrag(vp, i);
    }
    constexpr int NH = 2 * NSL;  // half-slots, each followed by softmax slices
#pragma unroll
    for (int i = 0; i < NSL; ++i) {
      // K.Q^T, then a slice of the softmax
      if (i < QF) {
        sout = QK::mma(kf[i], qf[i], sout);
        if (i + PFK < QF)
          kf[i + PFK] = kfrag(kp, i + PFK);
        else if (PRE)
          kpre[i + PFK - QF] = kfrag(kpn, i + PFK - QF);
      }
#pragma unroll
      for (int ch = (2 * i) * NCHUNK / NH; ch < (2 * i + 1) * NCHUNK / NH; ++ch) chunk(ch);
      __builtin_amdgcn_sched_barrier(0);
      // P.V, then a slice of the softmax
      if (i < NPV) {
        acc[i % NDB] = Mma<T>::mma(vf[i], pin[i / NDB], acc[i % NDB]);
        if (i + PFV < NPV)
          vf[i + PFV] = vfrag(vp, i + PFV);
        else if (PRE)
          vpre[i + PFV - NPV] = vfrag(vpn, i + PFV - NPV);
      }
      // the previous block's rounded sums, spread over the block
      if (LRM && (i == NSL / 4 || i == NSL / 2 + NSL / 4)) lr_mma(pin[i == NSL / 4 ? 0 : 1]);
#pragma unroll
      for (int ch = (2 * i + 1) * NCHUNK / NH; ch < (2 * i + 2) * NCHUNK / NH; ++ch) chunk(ch);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (fresh || __builtin_amdgcn_ballot_w64(over) != 0) {
      // rare: the reference moves, and the block is exponentiated again
      move_reference(sin);
      softmax_block(sin, pw, psa, rsa);
      // under the window mask a block may hide every key of some row: the
      // wave stays on this path until each of its rows has a reference
      fresh = MASKED ? __builtin_amdgcn_ballot_w64(m_use == -INFINITY) != 0 : false;
    }
    l += psa;
    if (!LRM) lr += rsa;
    pout[0] = __builtin_bit_cast(frag, pw[0]);
    pout[1] = __builtin_bit_cast(frag, pw[1]);
  }

  // Block b of this wave (its tile-local half and ring stages given): full
  // step, masked step (causal diagonal / key tail), or nothing past the
  // wave's last block (the caller runs the drain, the P.V of that last
  // block, after the ring loop).
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
      const int k0 = key0(b);
      if (needs_mask(k0)) mask(sin, k0);
      block_step(kp, vp, sin, sout, pin, pout);
    }
  }
  // The same for blocks chained by read-ahead (every block of the wave, no
  // drain): the first fragments of this block are in kpre/vpre, and those of
  // the next block (stages and halves given) are read during this one.  A
  // block past lastb (causal) does nothing; every later one is past it too.
  template <bool ODD>
  __device__ __forceinline__ void block_pre(const lds_char *ring, int b, int lastb, int vst,
                                            int vhalf, int kst, int khalf, int vst_n,
                                            int vhalf_n, int kst_n, int khalf_n) {
    f32x16 &sin = ODD ? S1 : S0;
    f32x16 &sout = ODD ? S0 : S1;
    frag(&pin)[2] = ODD ? P0 : P1;
    frag(&pout)[2] = ODD ? P1 : P0;
    if (b <= lastb) {
      const int k0 = key0(b);
      if (needs_mask(k0)) mask(sin, k0);
      block_step<true>(kptr(ring, kst, khalf), vptr(ring, vst, vhalf), sin, sout, pin, pout,
                       kptr(ring, kst_n, khalf_n), vptr(ring, vst_n, vhalf_n));
    }
  }
  // Reads the first fragments of a block ahead (the first of a chain).
  __device__ __forceinline__ void read_ahead(const lds_char *ring, int vst, int vhalf, int kst,
                                             int khalf) {
#pragma unroll
    for (int i = 0; i < (PFK > PFV ? PFK : PFV); ++i) {
      if (i < PFK) kpre[i] = kfrag(kptr(ring, kst, khalf), i);
      if (i < PFV) vpre[i] = vfrag(vptr(ring, vst, vhalf), i);
    }
  }
};

// Partial result of one split part, per row: O_p = acc / lr (fp32, D values),
// and the statistics (m, l, lr, 0) as one 16-byte record, m being the base-2
// exponent reference.  A row that saw no
// key in this part has l = lr = 0, m = -inf and O_p = 0.
template <int D>
__device__ __forceinline__ void epilogue_partial(const f32x16 (&acc)[(D + 31) / 32], float m,
                                                 float l, float lr, float *ws_o,
                                                 float *ws_s, int row, int g,
                                                 float osc = 1.f, int cb = 0,
                                                 int ce = (D + 31) / 32, bool stats = true) {
  const float lt = l + __shfl_xor(l, 32);
  const float lrt = lr;  // already the whole row's sum
  // O_p carries the factor osc: the combine is linear in the O_p
  const float inv = (lrt > 0.f ? 1.0f / lrt : 0.f) * osc;
  store_row<float, (D + 31) / 32>(acc, inv, ws_o + (size_t)row * D, g, D, cb, ce);
  if (stats && g == 0) {
    const f32x4 st = {lrt > 0.f ? m : -INFINITY, lt, lrt, 0.f};
    *reinterpret_cast<f32x4 *>(ws_s + row * 4) = st;
  }
}

// ---------------------------------------------------------------------------
// Eight waves per workgroup, two per SIMD, in one of two layouts:
//
// * PAIR = false (256 query rows, 32 per wave): every wave runs both 32-key
//   blocks of each 64-key ring step, so the per-step costs (the barrier, the
//   DMA issue, the loop) are shared by two blocks, and the two waves of a
//   SIMD fill each other's idle issue slots.
// * PAIR = true (128 query rows): waves w and w + 4 hold the same 32 rows
//   (group w % 4, on the same SIMD) and split the key blocks by parity, one
//   block per wave per step; at the end the pair's running statistics and
//   accumulators are combined through LDS with the online-softmax rescaling
//   (2^(m_i - M)) and the even wave writes O and L.  Twice as many
//   workgroups for the same rows: used when query tiles are few.
constexpr int kWaves8 = 8;
constexpr int kThreads8 = kWave * kWaves8;

template <bool PAIR>
struct QRows {
  static constexpr int value = PAIR ? 32 * kWaves8 / 2 : 32 * kWaves8;
};
static_assert(QRows<true>::value == kPairRows && QRows<false>::value == kGridRows &&
                  kBN == kKeys,
              "tile shapes of the stream schedule");

// DMA of one ring unit (one K tile, one V tile): each tile's 16-byte-per-lane
// load instructions are dealt to the eight waves round-robin, K in the first
// KJ slots of every wave and V in the next VJ, each padded to a multiple of
// eight with dummy loads (out of range, so they fetch nothing and write
// zeros into a 1 KB LDS scratch line).  With issue(), every wave issues the
// same number of loads per unit, so one vmcnt value describes "the youngest
// unit may still be in flight" for all of them, and each slot's tile (K or
// V) is known at compile time.  issue_k / issue_v (the pair-split loop,
// whose waits are for every load) skip the padding.  Measured on MI355X:
// skipping it in the pair-split loop +1.7%; in the 256-row loop, where the
// waits then need each wave's own count (a scalar branch per step), +-0 at
// D = 128 and 1-5% slower at D = 16-64.
template <typename T, int D, typename KT = T, typename LAY = PipeLayout<T, D, KT>>
struct Dma8 {
  typedef LAY L;
  static constexpr int KJ = (L::K_INS + kWaves8 - 1) / kWaves8;
  static constexpr int VJ = (L::V_INS + kWaves8 - 1) / kWaves8;
  static constexpr int PER_WAVE = KJ + VJ;
  static constexpr int SCRATCH = L::LDS_BYTES;
  static constexpr int LDS_BYTES = L::LDS_BYTES + kWave * 16;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");

  uint32_t src[PER_WAVE];    // per-lane byte offset in tile 0 (or out of range)
  uint32_t lbase[PER_WAVE];  // LDS destination in stage 0 (wave-uniform)
  uint32_t lstride[PER_WAVE];

  __device__ __forceinline__ void init(uint32_t ring_addr, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const bool isk = j < KJ;
      const int i = (isk ? j : j - KJ) * kWaves8 + wave;  // instruction within the tile
      uint32_t lb, ls;
      if (i < (isk ? L::K_INS : L::V_INS)) {
        lb = ring_addr + (isk ? 0u : (uint32_t)L::V_OFF) + (uint32_t)i * kWave * 16;
        ls = isk ? L::K_BYTES : L::V_BYTES;
        src[j] = dma_src(i, lane, isk ? L::SK : L::SV, isk ? L::KRB : D * (int)sizeof(T));
      } else {
        lb = ring_addr + SCRATCH;
        ls = 0;
        src[j] = kOutOfRange;
      }
      // wave-uniform: keep them in scalar registers
      lbase[j] = __builtin_amdgcn_readfirstlane(lb);
      lstride[j] = __builtin_amdgcn_readfirstlane(ls);
    }
  }

  // K tile `ktile` into stage kst, V tile `vtile` into stage vst (absolute
  // tile indices of the head's slice).
  __device__ __forceinline__ void issue(u32x4 k_rs, u32x4 v_rs, int ktile, int kst,
                                        int vtile, int vst) const {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const bool isk = j < KJ;
      const uint32_t lds = lbase[j] + (uint32_t)(isk ? kst : vst) * lstride[j];
      const uint32_t off =
          src[j] + (isk ? (uint32_t)ktile * L::K_TILE_GLOBAL : (uint32_t)vtile * L::V_TILE_GLOBAL);
      dma16(isk ? k_rs : v_rs, lds, off);
    }
  }
  // The K tile alone, or the V tile alone, without the padding loads: each
  // wave issues only its own instructions of the tile (lstride = 0 marks a
  // padding slot, wave-uniform), so the per-wave counts differ and only
  // waits for every load (vmcnt(0)) or for a count taken from kloads() may
  // follow.  Measured on MI355X: +1.4% at B8 N4096 D128 causal, +2.7%
  // non-causal (the padding loads wrote 11 of the unit's 48 KB of LDS).
  __device__ __forceinline__ void issue_k(u32x4 k_rs, int ktile, int kst) const {
#pragma unroll
    for (int j = 0; j < KJ; ++j)
      if (lstride[j] != 0)
        dma16(k_rs, lbase[j] + (uint32_t)kst * lstride[j],
              src[j] + (uint32_t)ktile * L::K_TILE_GLOBAL);
  }
  __device__ __forceinline__ void issue_v(u32x4 v_rs, int vtile, int vst) const {
#pragma unroll
    for (int j = KJ; j < PER_WAVE; ++j)
      if (lstride[j] != 0)
        dma16(v_rs, lbase[j] + (uint32_t)vst * lstride[j],
              src[j] + (uint32_t)vtile * L::V_TILE_GLOBAL);
  }
  // This wave's instructions of one K tile (issue_k).
  __device__ __forceinline__ int kloads() const {
    int n = 0;
#pragma unroll
    for (int j = 0; j < KJ; ++j) n += lstride[j] != 0 ? 1 : 0;
    return n;
  }
};

// MASKED (256-row layout only): the item's key tiles are the list kl (its
// kt0, kt1 index the list), scores follow the window rule mk.
// KT: the Q and K element type (T, or bytes holding e4m3 values for the
// FP8 score product); V is T.  osc multiplies O (the FP8 path's V descale).
template <typename T, typename OT, int D, bool CAUSAL, bool PAIR, bool MASKED = false,
          typename KT = T>
__device__ __forceinline__ void pipe8_run(const KT *__restrict__ q, const KT *__restrict__ k,
                                          const T *__restrict__ v, OT *__restrict__ o,
                                          float *__restrict__ lse, float *__restrict__ ws,
                                          int Nq, int Nk, float c, int negate,
                                          const PipeItem it, int nslots, const Mask mk = Mask{},
                                          const KeyList kl = KeyList{}, float osc = 1.f) {
  static_assert(!(MASKED && PAIR), "the window mask runs in the 256-row layout");
  typedef Pipe<T, OT, D, CAUSAL, MASKED, KT> P;
  typedef typename P::L L;
  typedef typename P::frag frag;
  typedef Dma8<T, D, KT> DM;
  constexpr int QPC = P::QK::FB / 16;  // 16-byte pieces of a K.Q^T operand per lane
  constexpr int UNIT = DM::PER_WAVE;
  constexpr int QT = QRows<PAIR>::value;
  __shared__ __attribute__((aligned(16))) char ring_[DM::LDS_BYTES];
  lds_char *ring = (lds_char *)ring_;
  const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;

  P s;
  // Opaque per call: a workgroup running several items recomputes the
  // lane-derived addresses for each one instead of keeping them in
  // registers across items (there are none to spare).
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = PAIR ? (wave & 3) : wave;  // query group (32 rows)
  const int h = PAIR ? (wave >> 2) : 0;     // block parity (PAIR)
  s.lane = tid & 63;
  s.wave = qg;
  s.l32 = s.lane & 31;
  s.g = s.lane >> 5;
  s.Nk = Nk;
  s.c = c;
  s.kbase = (uint32_t)(s.l32 * L::SK * 16 + s.g * P::QK::FB);
  s.osc = osc;
  {
    const int G = s.lane >> 4, s16 = s.lane & 15;
    const int row = 4 * (G >> 1) + (s16 >> 2);
    const int col = 16 * (G & 1) + 4 * (s16 & 3);  // element within the 32-wide d block
    s.vbase = (uint32_t)L::V_OFF + (uint32_t)row * L::SV * 16 + (uint32_t)col * 2;
  }
  s.qw = it.q0 + qg * 32;
  s.my_q = s.qw + s.l32;
  s.mk = mk;
  s.kl = kl;
  const size_t qoff = (size_t)it.bh * Nq * D;
  const size_t koff = (size_t)it.bh * Nk * D;
  const u32x4 q_rs = raw_rsrc(q + qoff, (uint32_t)Nq * D * sizeof(KT));
  const u32x4 k_rs = raw_rsrc(k + koff, (uint32_t)Nk * D * sizeof(KT));
  const u32x4 v_rs = raw_rsrc(v + koff, (uint32_t)Nk * D * sizeof(T));
  DM dm;
  dm.init(ring_addr, wave, s.lane);

  const int kt0 = it.kt0;
  const int ntiles = it.kt1 - it.kt0;
  // last 32-key block (absolute index; MASKED: index in the list) this
  // query group needs in this item
  int lastb = CAUSAL ? min(2 * it.kt1 - 1, s.qw / 32) : 2 * it.kt1 - 1;
  if constexpr (MASKED && CAUSAL) {
    // The group's last visible key is its diagonal, 0-3 key tiles before the
    // end of the tile's list (which ends at the tile's last query): the
    // drain after the loop finds its V tile still in the ring.  Without the
    // causal rule every group runs to the end of the list (its blocks past
    // its band are all hidden): a group's band may end four key tiles
    // before the list does, or many more when the tile holds global queries,
    // and its V tile would have left the ring by the drain.
    const int lk = min(Nk - 1, s.qw + 31);
    const int at = lk / kBN;
    int vb;
    if (at < kl.n1)
      vb = 2 * at + ((lk >> 5) & 1);
    else if (at >= kl.b0)
      vb = 2 * (at - kl.b0 + kl.n1) + ((lk >> 5) & 1);
    else
      vb = 2 * kl.n1 - 1;  // in the gap between the ranges: the global tiles' last block
    lastb = min(2 * it.kt1 - 1, vb);
  }

  // Q first: its loads are the oldest in flight, so the prologue wait for
  // the first K/V unit covers them too.
  u32x4 qraw[P::QF * QPC];
#pragma unroll
  for (int f = 0; f < P::QF; ++f)
#pragma unroll
    for (int j = 0; j < QPC; ++j)
      qraw[f * QPC + j] =
          load16_async(q_rs, (uint32_t)s.my_q * L::KRB + (2 * f + s.g) * P::QK::FB + 16 * j);

  // The first P.V of a wave belongs to the block before the item (P = 0)
  // and reads V stage 3 (rows 32..63, and with PAIR also rows 0..31), which
  // no load has written yet: clear it so that 0 * stale LDS cannot give NaN.
  // Everything else the kernel reads was written by a load (rows past Nk by
  // the bounds check, as zero).
  {
    constexpr int Z0 = L::V_OFF + 3 * L::V_BYTES + (PAIR ? 0 : 32 * L::SV * 16);
    constexpr int ZN = (PAIR ? 64 : 32) * L::SV;  // 16-byte chunks
    for (int i = tid; i < ZN; i += kThreads8)
      *(__attribute__((address_space(3))) u32x4 *)(ring + Z0 + i * 16) = u32x4{};
  }

  // Issue units: unit 0 = (K0,V0), 1 = (K1,V1), 2 = (K2,V2) in the
  // prologue, then step r issues unit r+3 = (K(r+3), V(r+2)) (relative
  // tiles; tile j lives in ring stage j % 4).  Unit j >= 1 is issued only
  // when j <= ntiles: nothing is fetched past the item except one K tile
  // whose scores are never used.  Every wave issues the same number of loads
  // per unit, so "the youngest unit may be in flight" is one vmcnt value.
  if constexpr (!PAIR) {
    dm.issue(k_rs, v_rs, s.kt_act(kt0), 0, s.kt_act(kt0), 0);
    dm.issue(k_rs, v_rs, s.kt_act(kt0 + 1), 1, s.kt_act(kt0 + 1), 1);
    if (ntiles >= 2) {
      dm.issue(k_rs, v_rs, s.kt_act(kt0 + 2), 2, s.kt_act(kt0 + 2), 2);
      ring_barrier<2 * UNIT>();
    } else {
      ring_barrier<UNIT>();
    }
  } else {
    // K tiles 0, 1, 2 and V tile 0; the loop's first barrier waits for all
    // of them, the prologue's for Q, K0 and V0 (this wave's loads of K1 and
    // K2 may be in flight)
    dm.issue_k(k_rs, kt0, 0);
    dm.issue_v(v_rs, kt0, 0);
    dm.issue_k(k_rs, kt0 + 1, 1);
    dm.issue_k(k_rs, kt0 + 2, 2);
    static_assert(DM::KJ <= 3, "ring_barrier_k2 range");
    ring_barrier_k2(dm.kloads());
  }
  // a negative scale flips the sign bit of every Q element
  constexpr uint32_t SIGN = sizeof(KT) == 1 ? 0x80808080u : 0x80008000u;
#pragma unroll
  for (int f = 0; f < P::QF * QPC; ++f) {
    asm volatile("" : "+v"(qraw[f]));  // Q is read only after the wait above
    if (negate) qraw[f] ^= u32x4{SIGN, SIGN, SIGN, SIGN};
  }
#pragma unroll
  for (int f = 0; f < P::QF; ++f) {
    if constexpr (QPC == 1) {
      s.qf[f] = __builtin_bit_cast(typename P::kfrag_t, qraw[f]);
    } else {
      const u32x4 a = qraw[2 * f], b = qraw[2 * f + 1];
      const i32x8 x = {(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                       (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
      s.qf[f] = __builtin_bit_cast(typename P::kfrag_t, x);
    }
  }

#pragma unroll
  for (int db = 0; db < P::NDB; ++db) s.acc[db] = f32x16{};
  s.m_use = -INFINITY;
  s.nm = 0.f;
  s.fresh = true;
  s.l = 0.f;
  s.lr = 0.f;
  s.lracc = f32x16{};
  s.P1[0] = frag{};  // P.V of the block before the first adds nothing
  s.P1[1] = frag{};
  s.qk(s.kptr(ring, 0, h), s.S0);

  if constexpr (!PAIR) {
    // Step r reads K tiles r, r+1 and V tiles r-1, r (relative):
    //   block 2r  : P.V(V tile r-1, rows 32..63), K.Q^T(K tile r, rows 32..63)
    //   block 2r+1: P.V(V tile r, rows 0..31),    K.Q^T(K tile r+1, rows 0..31)
    // K(r+1) and V(r) belong to units <= r+1, issued at least two steps
    // earlier; unit r+2 (issued in step r-1, if at all) may still be in
    // flight.  Step r requests unit r+3: K(r+3) into the stage of K(r-1) and
    // V(r+2) into the stage of V(r-2), both last read in step r-1.  Every
    // wave runs every step so that the loads and barriers line up.
    //
    // Each block reads the first fragments of the next one during its last
    // MFMAs (both tiles are in LDS by then: block 2r+1 reads K(r+1), V(r),
    // and block 2r+2 of the next step the other halves of the same tiles),
    // so a block never starts on a fresh LDS round trip.  Those reads are
    // the wave's youngest LDS accesses at the next barrier, which lets them
    // stay in flight: they touch neither stage the next unit overwrites.
    constexpr int RA = P::PFK * QPC + 2 * P::PFV;  // LDS reads of one read-ahead
    s.read_ahead(ring, kStages - 1, 1, 0, 1);
    for (int r = 0; r < ntiles; ++r) {
      ring_barrier_sel<UNIT, RA>(r + 2 <= ntiles);
      if (r + 3 <= ntiles)
        dm.issue(k_rs, v_rs, s.kt_act(kt0 + r + 3), (r + 3) & (kStages - 1),
                 s.kt_act(kt0 + r + 2), (r + 2) & (kStages - 1));
      const int st0 = r & (kStages - 1);
      const int stm = (r + kStages - 1) & (kStages - 1);
      const int st1 = (r + 1) & (kStages - 1);
      const int b = 2 * (kt0 + r);
      s.template block_pre<false>(ring, b, lastb, stm, 1, st0, 1, st0, 0, st1, 0);
      s.template block_pre<true>(ring, b + 1, lastb, st0, 0, st1, 0, st0, 1, st1, 1);
    }
    // Drain: P.V of the wave's last block (its P sits in P0 for an even
    // block, P1 for an odd one).  The last step's wait covered every unit
    // issued (units <= ntiles), and no unit overwrites the V tiles of the
    // item's last four steps, where a wave's last block always lies.
    if (lastb >= 2 * kt0) {
      const int rl = (lastb >> 1) - kt0;
      frag pl[2];
      pl[0] = (lastb & 1) ? s.P1[0] : s.P0[0];
      pl[1] = (lastb & 1) ? s.P1[1] : s.P0[1];
      s.pv(s.vptr(ring, rl & (kStages - 1), lastb & 1), pl);
    }
  } else {
    // Step r: this wave's block b = 2(kt0 + r) + h.  It reads K tile r+1
    // (half h, for the K.Q^T of block b+2) and V tile r-1 (half h, for the
    // P.V of block b-2).  Steps run in pairs (r even, r+1) under one barrier,
    // so that the barrier and the DMA issue serve two blocks per wave: the
    // pair reads K tiles r+1, r+2 and V tiles r-1, r, all issued before the
    // barrier, which waits for every load in flight; after it the wave
    // issues K tiles r+3, r+4 and V tiles r+1, r+2 into the four stages that
    // the pair does not read (their previous tiles were last read before
    // the barrier).  K tiles up to ntiles (one past the item: scores that
    // are never used) and V tiles below ntiles are fetched.  S and P
    // alternate registers from step to step.
    auto step = [&](int r, auto odd) {
      if ((r & 1) == 0) {
        ring_barrier<0>();
        if (r + 3 <= ntiles) dm.issue_k(k_rs, kt0 + r + 3, (r + 3) & (kStages - 1));
        if (r + 4 <= ntiles) dm.issue_k(k_rs, kt0 + r + 4, r & (kStages - 1));
        if (r + 1 < ntiles) dm.issue_v(v_rs, kt0 + r + 1, (r + 1) & (kStages - 1));
        if (r + 2 < ntiles) dm.issue_v(v_rs, kt0 + r + 2, (r + 2) & (kStages - 1));
      }
      const int b = 2 * (kt0 + r) + h;
      s.template block<decltype(odd)::value>(ring, b, lastb, (r + kStages - 1) & (kStages - 1),
                                                h, (r + 1) & (kStages - 1), h);
    };
    for (int r = 0; r < ntiles; r += 2) {
      step(r, std::false_type{});
      if (r + 1 < ntiles) step(r + 1, std::true_type{});
    }
    // Drain: P.V of this wave's last block, made in step rl: its P sits in
    // P0 or P1 by the parity of rl.  Its V tile may have been issued after
    // the last barrier: wait for every load first.
    ring_barrier<0>();
    const int mylast = lastb - ((lastb - h) & 1);  // last block of parity h
    if (mylast >= 2 * kt0 + h) {
      const int rl = mylast / 2 - kt0;
      frag pl[2];
      pl[0] = (rl & 1) ? s.P1[0] : s.P0[0];
      pl[1] = (rl & 1) ? s.P1[1] : s.P0[1];
      s.pv(s.vptr(ring, rl & (kStages - 1), h), pl);
    }
  }
  wait_vmcnt<0>();  // no DMA may outlive the ring
  ring_barrier<0>();  // every wave is done with the ring

  // lr: the row's whole rounded sum (every lane of a query holds it)
  float M = s.m_use, l = s.l, lr = s.lr_total();
  // PAIR: each wave of the pair stores half of the head-dim columns (blocks
  // [cb, cb + NDB / 2)); otherwise one wave stores them all.
  int cb = 0, ce = P::NDB;
  if constexpr (PAIR) {
    // Combine the pair, each wave the half of the columns it stores: a wave
    // hands the partner's half of acc and its (m, l, lr) over, and rescales
    // its own half with the partner's (the online-softmax update applied to
    // two partial states).
    static_assert(P::NDB % 2 == 0, "pair split of the columns");
    constexpr int HB = P::NDB / 2;                 // column blocks per wave
    constexpr int XW = (HB * 4 + 1) * kWave * 16;  // bytes one wave hands over
    lds_char *xw = ring + (uint32_t)(2 * qg + h) * XW;      // written by this wave
    lds_char *xr = ring + (uint32_t)(2 * qg + 1 - h) * XW;  // written by the partner
    cb = h * HB;
    ce = cb + HB;
    // the partner's blocks (static indices: acc stays in registers)
    auto hand = [&](const int ob) {
#pragma unroll
      for (int j = 0; j < HB; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 x = {s.acc[ob + j][4 * r4], s.acc[ob + j][4 * r4 + 1],
                           s.acc[ob + j][4 * r4 + 2], s.acc[ob + j][4 * r4 + 3]};
          *(__attribute__((address_space(3))) f32x4 *)(xw + ((j * 4 + r4) * kWave + s.lane) * 16) = x;
        }
    };
    if (h == 0)
      hand(HB);
    else
      hand(0);
    {
      const f32x4 st = {s.m_use, s.l, lr, 0.f};
      *(__attribute__((address_space(3))) f32x4 *)(xw + (HB * 4 * kWave + s.lane) * 16) = st;
    }
    ring_barrier<0>();
    const f32x4 st =
        *(const __attribute__((address_space(3))) f32x4 *)(xr + (HB * 4 * kWave + s.lane) * 16);
    // A wave that saw no key of a row (its blocks lie past the row under the
    // causal mask, or the item starts there) has m = -inf, l = 0, acc = 0
    // and weight 0; when neither wave saw one the row's partial is empty
    // (l = 0).  Both waves form M, l and lr, and their halves of acc, by
    // the same expressions with the even wave's terms first, so that the two
    // agree bit for bit.
    M = fmaxf(s.m_use, st[0]);
    const float a0 = s.m_use == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s.m_use - M);
    const float a1 = st[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st[0] - M);
    f32x4 x[HB][4];
#pragma unroll
    for (int j = 0; j < HB; ++j)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        x[j][r4] = *(const __attribute__((address_space(3))) f32x4 *)(
            xr + ((j * 4 + r4) * kWave + s.lane) * 16);
    if (h == 0) {
      l = __builtin_fmaf(s.l, a0, st[1] * a1);
      lr = __builtin_fmaf(lr, a0, st[2] * a1);
#pragma unroll
      for (int j = 0; j < HB; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s.acc[j][4 * r4 + e] =
                __builtin_fmaf(s.acc[j][4 * r4 + e], a0, x[j][r4][e] * a1);
    } else {
      l = __builtin_fmaf(st[1], a1, s.l * a0);
      lr = __builtin_fmaf(st[2], a1, lr * a0);
#pragma unroll
      for (int j = 0; j < HB; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s.acc[HB + j][4 * r4 + e] =
                __builtin_fmaf(x[j][r4][e], a1, s.acc[HB + j][4 * r4 + e] * a0);
    }
    // The ring is free for the workgroup's next item once every read of the
    // exchange area is done.
    ring_barrier<0>();
  }

  const bool stats = !PAIR || h == 0;  // the wave that writes L (or the record)
  if (it.slot < 0) {
    epilogue<D, OT>(s.acc, M, l, o, lse, it.bh, Nq, s.my_q, s.g, lr, osc, cb, ce, stats);
  } else {
    float *ws_o = ws + (size_t)it.slot * QT * D;
    float *ws_s = ws + (size_t)nslots * QT * D + (size_t)it.slot * QT * 4;
    epilogue_partial<D>(s.acc, M, l, lr, ws_o, ws_s, s.my_q - it.q0, s.g, osc, cb, ce, stats);
  }
}

// Key tiles of the query tile at rows [q0, q0 + QT) under the window rule
// mk (window <= max(Nq, Nk) as clamped by the host, so nothing overflows):
// the global tokens' key tiles (causal: keys j <= the tile's last query),
// then the band's, [q0 - window + 1, last query (+ window - 1 non-causal)];
// every key tile for a non-causal tile holding global queries.  *n is the
// list's length (0: the tile sees no key).
__device__ __forceinline__ KeyList key_list(const Mask &mk, int q0, int QT, int Nq, int Nk,
                                            int *n) {
  const int qlast = min(q0 + QT, Nq) - 1;
  const int nkt = (Nk + kBN - 1) / kBN;
  if (!mk.causal && q0 < mk.nglobal) {
    *n = nkt;
    return {nkt, nkt};
  }
  const int gend = mk.causal ? min(min(mk.nglobal, Nk), qlast + 1) : min(mk.nglobal, Nk);
  const int n1 = (gend + kBN - 1) / kBN;
  const int blo = max(0, q0 - mk.window + 1);
  const int bhi = mk.causal ? min(Nk - 1, qlast) : min(Nk - 1, qlast + mk.window - 1);
  if (blo > bhi) {  // no band key
    *n = n1;
    return {n1, n1};
  }
  const int b0 = blo / kBN, b1 = bhi / kBN + 1;
  if (b0 <= n1) {  // the ranges meet: one range from tile 0
    *n = max(n1, b1);
    return {*n, *n};
  }
  *n = n1 + (b1 - b0);
  return {n1, b0};
}

// One workgroup per (batch*head, query tile), longest causal tiles first.
// MASKED: the tile's key tiles are its key_list under the window rule mk; a
// tile that sees no key writes O = 0 and L = -inf.
template <typename T, typename OT, int D, bool CAUSAL, bool PAIR, bool MASKED = false,
          typename KT = T>
__global__ __launch_bounds__(kThreads8) void fa_fwd_pipe8(
    const KT *__restrict__ q, const KT *__restrict__ k, const T *__restrict__ v,
    OT *__restrict__ o, float *__restrict__ lse, int Nq, int Nk, int BH, int nqt,
    float c, int negate, Mask mk, float osc, float *__restrict__ ws, int nsp, int S) {
  FA_DBG_BEGIN();
  constexpr int QT = QRows<PAIR>::value;
  WorkItem wi = work_item(BH, nqt, CAUSAL, QT);
  if constexpr (MASKED) {
    // Split (S > 1, without the causal rule): the first nsp * S units are
    // S parts of each of the tiles [0, nsp) of every slice (those holding
    // global queries, whose lists hold every key tile); part p takes list
    // entries [p n / S, (p + 1) n / S) and leaves its partial result in
    // workspace slot (bh * nsp + t) * S + p for fa_merge_masked_split.
    const int u = blockIdx.x / BH;
    int p = -1;
    if (u < nsp * S) {
      p = u % S;
      wi.q0 = (u / S) * QT;
    } else if (nsp > 0) {
      wi.q0 = (u - nsp * S + nsp) * QT;
    }
    int n;
    const KeyList kl = key_list(mk, wi.q0, QT, Nq, Nk, &n);
    const int nslots = BH * nsp * S;
    if (p >= 0) {
      const int e0 = (int)((int64_t)p * n / S), e1 = (int)((int64_t)(p + 1) * n / S);
      const int slot = (wi.bh * nsp + wi.q0 / QT) * S + p;
      if (e0 >= e1) {  // an empty part: a partial result with no key
        float *wo = ws + (size_t)slot * QT * D;
        float *wst = ws + (size_t)nslots * QT * D + (size_t)slot * QT * 4;
        for (int i = threadIdx.x; i < QT * D; i += kThreads8) wo[i] = 0.f;
        for (int i = threadIdx.x; i < QT; i += kThreads8)
          *reinterpret_cast<f32x4 *>(wst + 4 * i) = f32x4{-INFINITY, 0.f, 0.f, 0.f};
        return;
      }
      const PipeItem it = {wi.bh, wi.q0, e0, e1, slot};
      pipe8_run<T, OT, D, CAUSAL, PAIR, true>(q, k, v, o, lse, ws, Nq, Nk, c, negate, it,
                                              nslots, mk, kl);
      return;
    }
    if (n == 0) {
      const int rows = min(QT, Nq - wi.q0);
      const size_t r0 = (size_t)wi.bh * Nq + wi.q0;
      for (int i = threadIdx.x; i < rows * D; i += kThreads8) o[r0 * D + i] = (OT)0.f;
      for (int i = threadIdx.x; i < rows; i += kThreads8) lse[r0 + i] = -INFINITY;
      return;
    }
    const PipeItem it = {wi.bh, wi.q0, 0, n, -1};
    pipe8_run<T, OT, D, CAUSAL, PAIR, true>(q, k, v, o, lse, nullptr, Nq, Nk, c, negate, it, 0,
                                            mk, kl);
  } else {
    const int kend = CAUSAL ? min(Nk, wi.q0 + QT) : Nk;
    const PipeItem it = {wi.bh, wi.q0, 0, (kend + kBN - 1) / kBN, -1};
    pipe8_run<T, OT, D, CAUSAL, PAIR, false, KT>(q, k, v, o, lse, nullptr, Nq, Nk, c, negate,
                                                 it, 0, Mask{}, KeyList{}, osc);
  }
}

// Variable-length batches (page "FlashAttention-2实现与优化：高效注意力机制详解"
// §7, ragged input sequences): S sequences packed along the token axis of
// [H, T, D] tensors, sequence s at rows cu_q[s] .. cu_q[s+1] of every head
// (keys cu_k[s] .. cu_k[s+1]), each attending only to its own keys.  One
// workgroup per (tile rank, head, sequence), longest causal tiles first;
// workgroups past their sequence's end return at once.  A sequence is one
// slice for the pipelined kernel: its buffer resources end at the
// sequence's last row, so no read crosses into a neighbour.  Offsets are
// clamped to [0, T] (inconsistent offsets give wrong rows, never a read or
// write outside the tensors).  A sequence with queries and no keys gets
// O = 0 and L = -inf (the logarithm of an empty sum).  PAIR selects the
// pair-split 128-row layout (D = 128, few tiles) over the 256-row one.
//
// Split keys (NC > 1, the sequence parallelism of page "FlashAttention技术
// 演进全景图" §3.2 applied per sequence): a tile whose key range spans more
// than KC 64-key tiles is cut into chunks of KC, one workgroup each, which
// write (m, l, lr) and the normalised accumulator to workspace slot
// varlen_slot(...) for fa_merge_varlen; shorter tiles write O and L at once.
// Without it the longest sequence's last tile, run by one workgroup, bounds
// the whole call.
__device__ __forceinline__ int varlen_slot(int h, int NT, int NC, int qa, int q0, int QT,
                                           int sq, int chunk) {
  // floor((qa + q0) / QT) + sq is distinct for every (sequence, tile) of a
  // head: within a sequence consecutive tiles step it by one, and a later
  // sequence starts past the earlier one's last row with a larger sq; it is
  // below ceil(Tq / QT) + S = NT
  return (h * NT + (qa + q0) / QT + sq) * NC + chunk;
}

template <typename T, typename OT, int D, bool CAUSAL, bool PAIR>
__global__ __launch_bounds__(kThreads8) void fa_fwd_varlen(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    OT *__restrict__ o, float *__restrict__ lse, const int *__restrict__ cu_q,
    const int *__restrict__ cu_k, int S, int H, int Tq, int Tk, int ntiles, float c,
    int negate, float *__restrict__ ws, int NC, int KC, int NT) {
  FA_DBG_BEGIN();
  constexpr int QT = QRows<PAIR>::value;
  const int chunk = blockIdx.x % NC;
  const int id = blockIdx.x / NC;
  // rank-major (longest causal tiles first); the slice index is rotated by
  // the rank so that one sequence's tiles are spread over the XCDs (the
  // dispatcher deals workgroup ids to the 8 XCDs round robin: without the
  // rotation, H*S a multiple of 8 would keep every sequence on one XCD)
  const int t = id / (H * S);
  const int hs = (id % (H * S) + t) % (H * S);
  const int h = hs / S, sq = hs % S;
  const int qt = CAUSAL ? ntiles - 1 - t : t;
  const int qa = max(0, min(cu_q[sq], Tq)), qb = max(qa, min(cu_q[sq + 1], Tq));
  const int ka = max(0, min(cu_k[sq], Tk)), kb = max(ka, min(cu_k[sq + 1], Tk));
  const int nq = qb - qa, nk = kb - ka;
  const int q0 = qt * QT;
  const size_t qo = (size_t)h * Tq + qa, ko = (size_t)h * Tk + ka;
  if (qt == ntiles - 1 && chunk == 0 && nq > ntiles * QT) {
    // rows past the last tile the grid covers (the sequence is longer than
    // the caller's max_seqlen_q): defined as NaN rather than left unwritten
    const float nan = __builtin_nanf("");
    for (int i = ntiles * QT * D + threadIdx.x; i < nq * D; i += kThreads8)
      o[qo * D + i] = (OT)nan;
    for (int i = ntiles * QT + threadIdx.x; i < nq; i += kThreads8) lse[qo + i] = nan;
  }
  if (q0 >= nq) return;  // workgroup-uniform, before any barrier
  if (nk == 0) {
    if (chunk != 0) return;
    const int rows = min(QT, nq - q0);
    for (int i = threadIdx.x; i < rows * D; i += kThreads8)
      o[(qo + q0) * D + i] = (OT)0.f;
    for (int i = threadIdx.x; i < rows; i += kThreads8) lse[qo + q0 + i] = -INFINITY;
    return;
  }
  const int kend = CAUSAL ? min(nk, q0 + QT) : nk;
  const int nkt = (kend + kBN - 1) / kBN;
  PipeItem it = {0, q0, 0, nkt, -1};
  int kc;
  const int nch = varlen_split(nkt, NC, KC, kc);
  if (nch > 1) {  // split: this workgroup's chunk of the key tiles
    if (chunk >= nch) return;  // every chunk below nch holds key tiles
    it.kt0 = chunk * kc;
    it.kt1 = min(nkt, it.kt0 + kc);
    it.slot = varlen_slot(h, NT, NC, qa, q0, QT, sq, chunk);
  } else if (chunk != 0) {
    return;
  }
  pipe8_run<T, OT, D, CAUSAL, PAIR>(q + qo * D, k + ko * D, v + ko * D, o + qo * D, lse + qo,
                                    ws, nq, nk, c, negate, it, H * NT * NC);
}

// Chunk run by workgroup g: consecutive chunks go to one XCD (workgroups are
// dealt to the 8 XCDs round robin), so an XCD's workgroups share heads and
// their K/V in its L2.
__device__ __forceinline__ int chunk_of(int g, int G) {
  return (G % 8 == 0) ? (g % 8) * (G / 8) + g / 8 : g;
}

// Rows of a cut tile per combining workgroup (16 rows at D = 128, 64 at
// D = 64: measured fastest on MI355X; the workgroup's fixed cost of
// locating the tile weighs against fewer loads in flight per thread).
template <int D>
constexpr int merge_rows() { return D == 128 ? 16 : 64; }

// ---------------------------------------------------------------------------
// dQ of the backward pass on the forward's pipelined machinery.  The
// backward recomputes the probabilities from the saved logsumexp (page
// "解释FlashAttention的显存优化原理" §一.2(2)); for a 128-row query tile,
// with Q and dO held in registers like the forward's Q:
//
//     S^T  = K Q^T               (A: K rows from LDS, B: Q^T)
//     dP^T = V dO^T              (A: V rows from LDS, B: dO^T)
//     P = 2^(c s - L log2 e),  dS = P (dP - Dl)       (0 on hidden pairs)
//     dQ^T += K^T dS^T            (A: K^T by ds_read_b64_tr_b16, B: dS^T rounded to T)
//
// so one lane owns one query (L and Dl are per-lane scalars) and dS never
// leaves registers, as P in the forward.  K and V 64-key tiles stream through
// a four-stage DMA ring (buffer_load ... lds); K is read both by rows and
// transposed, so its row stride is the one that measured best for both in
// the backward's LDS blocks (19 slots at D = 128, 13 at D = 64), V keeps the
// forward's row stride.  Eight waves, two per SIMD: waves w and w + 4 hold
// query group w % 4 (32 rows) and take the even and odd 32-key blocks; their
// dQ^T partial sums are added through LDS at the end.  One workgroup per
// query tile, longest first under the causal mask.
template <typename T, int D>
struct DqLayout {
  static constexpr int KRB = D * (int)sizeof(T);
  static constexpr int SK = D == 128 ? 19 : 13;  // K rows (read both ways), 16-byte slots
  static constexpr int SV = KRB / 16 + 1;        // V rows (read by rows)
  static constexpr int K_BYTES = kBN * SK * 16;
  static constexpr int V_BYTES = kBN * SV * 16;
  static constexpr int K_INS = kBN * SK / kWave;
  static constexpr int V_INS = kBN * SV / kWave;
  static constexpr int V_OFF = kStages * K_BYTES;
  static constexpr int LDS_BYTES = kStages * (K_BYTES + V_BYTES);
  static constexpr uint32_t K_TILE_GLOBAL = kBN * KRB;
  static constexpr uint32_t V_TILE_GLOBAL = kBN * KRB;
  static_assert(LDS_BYTES <= 150 * 1024, "LDS");
};

// One item of the dQ kernel: key tiles [it.kt0, it.kt1) of the 128-row query
// tile at it.q0 of slice it.bh.  With it.slot < 0 the item is the whole tile
// and stores dQ (times scale, in OT); otherwise it writes its fp32 partial
// sum to workspace slot it.slot (128 rows of D), which fa_merge_dq8 adds up.
//
// Dl_i = <dO_i, O_i> is formed here from O and dO (each lane holds half of
// its query's row of both, the other half in lane l ^ 32), and the piece
// that starts at the tile's first key tile stores it to dl for the dK/dV
// pass, which runs after this one.
//
// MASKED: the local-window + global-token rule mk; the tile's key tiles are
// the list kl (its entries [kt0, kt1) are list indices), a block with no
// visible pair is skipped and the others test each score against the rule
// where some pair of the block is hidden.
template <typename T, typename OT, int D, bool CAUSAL, bool MASKED = false>
__device__ __forceinline__ void dq8_run(const T *__restrict__ q, const T *__restrict__ k,
                                        const T *__restrict__ v, const T *__restrict__ o,
                                        const T *__restrict__ dout,
                                        const float *__restrict__ lse, float *__restrict__ dl,
                                        OT *__restrict__ dq, float *__restrict__ ws, int Nq,
                                        int Nk, float c, float scale, const PipeItem it,
                                        bool reuse, const Mask mk = Mask{},
                                        const KeyList kl = KeyList{}) {
  typedef DqLayout<T, D> L;
  typedef Dma8<T, D, T, L> DM;
  typedef typename Mma<T>::frag frag;
  constexpr int QF = D / 16;   // MFMAs of S^T and of dP^T per 32-key block
  constexpr int NDB = D / 32;  // dQ^T blocks of 32 head-dim rows
  constexpr int QT = 128;
  __shared__ __attribute__((aligned(16))) char ring_[DM::LDS_BYTES];
  lds_char *ring = (lds_char *)ring_;
  const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;

  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = wave & 3, h = wave >> 2;
  const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int qw = it.q0 + qg * 32;
  const int my_q = qw + l32;
  const uint32_t kbase = (uint32_t)(l32 * L::SK * 16 + g * 16);
  const uint32_t vbase = (uint32_t)(L::V_OFF + l32 * L::SV * 16 + g * 16);
  uint32_t tbase;
  {
    const int G = lane >> 4, s16 = lane & 15;
    const int row = 4 * (G >> 1) + (s16 >> 2);
    const int col = 16 * (G & 1) + 4 * (s16 & 3);
    tbase = (uint32_t)(row * L::SK * 16 + col * 2);
  }
  const size_t qoff = (size_t)it.bh * Nq * D;
  const size_t koff = (size_t)it.bh * Nk * D;
  const u32x4 q_rs = raw_rsrc(q + qoff, (uint32_t)Nq * D * sizeof(T));
  const u32x4 do_rs = raw_rsrc(dout + qoff, (uint32_t)Nq * D * sizeof(T));
  const u32x4 o_rs = raw_rsrc(o + qoff, (uint32_t)Nq * D * sizeof(T));
  const u32x4 k_rs = raw_rsrc(k + koff, (uint32_t)Nk * D * sizeof(T));
  const u32x4 v_rs = raw_rsrc(v + koff, (uint32_t)Nk * D * sizeof(T));
  DM dm;
  dm.init(ring_addr, wave, lane);

  // rows past Nq: L = +inf gives P = 0
  const float l2 = my_q < Nq ? lse[(size_t)it.bh * Nq + my_q] * 1.4426950408889634f : INFINITY;
  float dd = 0.f;  // Dl of this lane's query (0 past Nq: O and dO read as zero)
  const int kt0 = it.kt0;
  const int ntiles = it.kt1 - it.kt0;
  // key tile of entry v (MASKED: of the list)
  auto kt_act = [&](int v) { return MASKED ? (v < kl.n1 ? v : kl.b0 + (v - kl.n1)) : v; };
  // last 32-key block (absolute; MASKED: in list order, the list's last)
  // with a key this wave's queries may see
  const int lastb = (CAUSAL && !MASKED) ? min(2 * it.kt1 - 1, (qw + 31) / 32) : 2 * it.kt1 - 1;

  u32x4 qraw[QF], draw[QF], oraw[QF];
#pragma unroll
  for (int f = 0; f < QF; ++f) {
    const uint32_t off = ((uint32_t)my_q * D + 16 * f + 8 * g) * sizeof(T);
    qraw[f] = load16_async(q_rs, off);
    draw[f] = load16_async(do_rs, off);
    oraw[f] = load16_async(o_rs, off);
  }
  dm.issue(k_rs, v_rs, kt_act(kt0), 0, kt_act(kt0), 0);
  if (ntiles > 1) dm.issue(k_rs, v_rs, kt_act(kt0 + 1), 1, kt_act(kt0 + 1), 1);
  frag qf[QF], dof[QF];
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  for (int r = 0; r < ntiles; ++r) {
    if ((r & 1) == 0) {
      // tiles r and r+1 have landed, and every wave is done with the stages
      // of tiles r-2 and r-1, which tiles r+2 and r+3 now take
      ring_barrier<0>();
      if (r + 2 < ntiles)
        dm.issue(k_rs, v_rs, kt_act(kt0 + r + 2), (r + 2) & 3, kt_act(kt0 + r + 2), (r + 2) & 3);
      if (r + 3 < ntiles)
        dm.issue(k_rs, v_rs, kt_act(kt0 + r + 3), (r + 3) & 3, kt_act(kt0 + r + 3), (r + 3) & 3);
      if (r == 0) {
        float part = 0.f;
#pragma unroll
        for (int f = 0; f < QF; ++f) {
          // read after the wait above
          asm volatile("" : "+v"(qraw[f]), "+v"(draw[f]), "+v"(oraw[f]));
          qf[f] = __builtin_bit_cast(frag, qraw[f]);
          dof[f] = __builtin_bit_cast(frag, draw[f]);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const f32x2 x = Mma<T>::unpack2(draw[f][w]), y = Mma<T>::unpack2(oraw[f][w]);
            part = __builtin_fmaf(x[0], y[0], part);
            part = __builtin_fmaf(x[1], y[1], part);
          }
        }
        dd = part + __shfl_xor(part, 32);
        if (it.kt0 == 0 && h == 0 && g == 0 && my_q < Nq) dl[(size_t)it.bh * Nq + my_q] = dd;
      }
    }
    const int b = 2 * (kt0 + r) + h;
    if (b > lastb) continue;  // wave-uniform; later blocks are past it too
    const int k0 = MASKED ? kt_act(b >> 1) * kBN + (b & 1) * 32 : 32 * b;
    if (MASKED && !mk.any(qw, qw + 31, k0, k0 + 31)) continue;  // wave-uniform
    const int st = r & 3;
    const lds_char *kp = ring + st * L::K_BYTES + h * 32 * L::SK * 16;
    const lds_char *vp = ring + st * L::V_BYTES + h * 32 * L::SV * 16;
    f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int f = 0; f < QF; ++f) {
      const frag kf = *(const __attribute__((address_space(3))) frag *)(kp + kbase + f * 32);
      const frag vf = *(const __attribute__((address_space(3))) frag *)(vp + vbase + f * 32);
      sc = Mma<T>::mma(kf, qf[f], sc);
      dp = Mma<T>::mma(vf, dof[f], dp);
    }
    // wave-uniform, and taken as a branch (the compiler had turned the
    // per-score test into selects on every block: +130 VALU per block)
    const int need_mask = __builtin_amdgcn_readfirstlane(
        (k0 + 32 > Nk) ||
                (MASKED ? !mk.all(qw, qw + 31, k0, k0 + 31) : (CAUSAL && k0 + 31 > qw))
            ? 1
            : 0);
    float ds[16];
    if (need_mask) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + acc_row(e, g);
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], c, -l2));
        if (key >= Nk || (MASKED ? !mk.visible(my_q, key) : (CAUSAL && key > my_q))) p = 0.f;
        ds[e] = p * (dp[e] - dd);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        ds[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], c, -l2)) * (dp[e] - dd);
    }
    frag dsb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 w = {Mma<T>::pack2(ds[8 * ks], ds[8 * ks + 1]),
                       Mma<T>::pack2(ds[8 * ks + 2], ds[8 * ks + 3]),
                       Mma<T>::pack2(ds[8 * ks + 4], ds[8 * ks + 5]),
                       Mma<T>::pack2(ds[8 * ks + 6], ds[8 * ks + 7])};
      dsb[ks] = __builtin_bit_cast(frag, w);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const lds_char *a0 = kp + tbase + ks * 16 * L::SK * 16 + db * 64;
        const u32x2 lo = read_tr16(a0);
        const u32x2 hi = read_tr16(a0 + 8 * L::SK * 16);
        const u32x4 raw = {lo[0], lo[1], hi[0], hi[1]};
        acc[db] = Mma<T>::mma(__builtin_bit_cast(frag, raw), dsb[ks], acc[db]);
      }
  }
  wait_vmcnt<0>();    // no DMA may outlive the ring
  ring_barrier<0>();  // every wave is done with the ring

  // the odd wave of each group hands its partial sums to the even one
  constexpr int NR = NDB * 4;
  lds_char *xch = ring + (uint32_t)qg * NR * kWave * 16;
  if (h == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 x = {acc[db][4 * r4], acc[db][4 * r4 + 1], acc[db][4 * r4 + 2],
                         acc[db][4 * r4 + 3]};
        *(__attribute__((address_space(3))) f32x4 *)(xch + ((db * 4 + r4) * kWave + lane) * 16) = x;
      }
  }
  ring_barrier<0>();
  if (h == 0) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 x = *(const __attribute__((address_space(3))) f32x4 *)(
            xch + ((db * 4 + r4) * kWave + lane) * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[db][4 * r4 + e] += x[e];
      }
    if (it.slot < 0) {
      if (my_q < Nq) store_row<OT, NDB>(acc, scale, dq + ((size_t)it.bh * Nq + my_q) * D, g, D);
    } else {
      store_row<float, NDB>(acc, 1.f, ws + ((size_t)it.slot * QT + (my_q - it.q0)) * D, g, D);
    }
  }
  // reuse: the ring (and the exchange area in it) is free for the
  // workgroup's next item once every read of the exchange area is done (the
  // stores need not be)
  if (reuse) ring_barrier<63, 0>();
}

// One workgroup per 128-row query tile, longest first under the causal mask.
// ws is never written here (every item is a whole tile); it is passed as an
// argument because this compiler crashes on the constant null pointer that
// the never-taken partial store would otherwise see.
//
// MASKED: the tile walks its key_list under the rule mk; a tile that sees no
// key gets dQ = 0 and Dl = 0 (nothing reads the Dl of such rows).
template <typename T, typename OT, int D, bool CAUSAL, bool MASKED = false>
__global__ __launch_bounds__(kThreads8) void fa_bwd_dq8(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ o, const T *__restrict__ dout, const float *__restrict__ lse,
    float *__restrict__ dl, OT *__restrict__ dq, float *__restrict__ ws, int Nq, int Nk, int BH,
    int nqt, float c, float scale, Mask mk, int nsp, int S) {
  FA_DBG_BEGIN();
  WorkItem wi = work_item(BH, nqt, CAUSAL, 128);
  if constexpr (MASKED) {
    // Split (S > 1, without the causal rule): the first nsp * S units are
    // S parts of each of the tiles [0, nsp) (those holding global queries,
    // whose lists hold every key tile); part p takes list entries
    // [p n / S, (p + 1) n / S) and leaves fp32 partial dQ in workspace slot
    // (bh * nsp + t) * S + p for fa_merge_dq8_split.  The first part that
    // holds entries starts at entry 0 and writes the row terms.
    const int u = blockIdx.x / BH;
    int p = -1;
    if (u < nsp * S) {
      p = u % S;
      wi.q0 = (u / S) * 128;
    } else if (nsp > 0) {
      wi.q0 = (u - nsp * S + nsp) * 128;
    }
    int n;
    const KeyList kl = key_list(mk, wi.q0, 128, Nq, Nk, &n);
    if (p >= 0) {
      const int e0 = (int)((int64_t)p * n / S), e1 = (int)((int64_t)(p + 1) * n / S);
      const int slot = (wi.bh * nsp + wi.q0 / 128) * S + p;
      if (e0 >= e1) {  // an empty part: zero partial sums
        float *w = ws + (size_t)slot * 128 * D;
        for (int i = threadIdx.x; i < 128 * D; i += kThreads8) w[i] = 0.f;
        return;
      }
      const PipeItem it = {wi.bh, wi.q0, e0, e1, slot};
      dq8_run<T, OT, D, CAUSAL, true>(q, k, v, o, dout, lse, dl, dq, ws, Nq, Nk, c, scale, it,
                                      false, mk, kl);
      return;
    }
    if (n == 0) {
      const int rows = min(128, Nq - wi.q0);
      const size_t r0 = (size_t)wi.bh * Nq + wi.q0;
      for (int i = threadIdx.x; i < rows * D; i += kThreads8) dq[r0 * D + i] = (OT)0.f;
      for (int i = threadIdx.x; i < rows; i += kThreads8) dl[r0 + i] = 0.f;
      return;
    }
    const PipeItem it = {wi.bh, wi.q0, 0, n, -1};
    dq8_run<T, OT, D, CAUSAL, true>(q, k, v, o, dout, lse, dl, dq, ws, Nq, Nk, c, scale, it,
                                    false, mk, kl);
  } else {
    const int kend = CAUSAL ? min(Nk, wi.q0 + 128) : Nk;
    const PipeItem it = {wi.bh, wi.q0, 0, (kend + kBN - 1) / kBN, -1};
    dq8_run<T, OT, D, CAUSAL>(q, k, v, o, dout, lse, dl, dq, ws, Nq, Nk, c, scale, it, false);
  }
}

// The stream-K schedule of the forward (128-row tiles): each workgroup walks
// its chunk of (query tile, 64-key tile) units; cut tiles leave partial sums.
template <typename T, typename OT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads8) void fa_bwd_dq8_stream(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ o, const T *__restrict__ dout, const float *__restrict__ lse,
    float *__restrict__ dl, OT *__restrict__ dq, float *__restrict__ ws, int Nq, int Nk,
    float c, float scale, StreamPlan sp, ChunkStarts cs) {
  FA_DBG_BEGIN();
  ChunkWalk cw;
  const int ch = chunk_of(blockIdx.x, sp.G);
  cw.init_at(sp, ch, cs.w[2 * ch], cs.w[2 * ch + 1]);
  PipeItem it;
  int t;
  while (cw.next(sp, CAUSAL, it, t)) {
    it.q0 = t * 128;
    dq8_run<T, OT, D, CAUSAL>(q, k, v, o, dout, lse, dl, dq, ws, Nq, Nk, c, scale, it, true);
  }
}

// Sums the partial dQ of each cut tile's pieces (in piece order) and stores
// scale times the sum: merge_rows<D>() rows of a tile per workgroup.
template <typename OT, int D>
__global__ __launch_bounds__(kThreads) void fa_merge_dq8(const float *__restrict__ ws,
                                                         OT *__restrict__ dq, int Nq,
                                                         float scale, CutList cuts) {
  constexpr int C4 = D / 4;
  constexpr int RPP = kThreads / C4;
  constexpr int ROWS = merge_rows<D>();
  constexpr int SPLIT = 128 / ROWS;
  constexpr int NR = ROWS / RPP;
  static_assert(NR >= 1 && ROWS % RPP == 0, "merge tiling");
  const uint32_t w0 = cuts.w[2 * (blockIdx.x / SPLIT)];
  const uint32_t w1 = cuts.w[2 * (blockIdx.x / SPLIT) + 1];
  const int bh = (int)(w0 & 0xffffu), t = (int)(w0 >> 16);
  const int np = cut_pieces(w1);
  const int c4 = threadIdx.x % C4;
  const int r0 = (blockIdx.x % SPLIT) * ROWS + threadIdx.x / C4;
  f32x4 acc[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kk = 0; kk < np; ++kk) {
    const size_t sl = (size_t)cut_slot(w1, kk);
#pragma unroll
    for (int i = 0; i < NR; ++i)
      acc[i] += *reinterpret_cast<const f32x4 *>(ws + (sl * 128 + r0 + i * RPP) * D + 4 * c4);
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int row = t * 128 + r0 + i * RPP;
    if (row < Nq) store4<OT>(dq + ((size_t)bh * Nq + row) * D + 4 * c4, acc[i] * scale);
  }
}

// ---------------------------------------------------------------------------
// dK and dV of the backward pass on the same machinery, the roles of keys and
// queries swapped: a workgroup holds 128 keys (K and V fragments in registers
// as the B operands of S = Q K^T and dP = dO V^T, one key per lane) and
// streams 64-row tiles of Q and dO through the DMA ring, with each tile's L
// and Dl; per 32-query block
//
//     P = 2^(c s - L log2 e),  dS = P (dP - Dl)          (0 on hidden pairs)
//     dV^T += dO^T P,   dK^T += Q^T dS                     (A: dO^T, Q^T by
//                                                          ds_read_b64_tr_b16)
//
// with P and dS from registers.  Waves w and w + 4 hold key group w % 4
// (32 keys) and take the two 32-row halves of each query tile; their sums
// are added through LDS at the end.  Q and dO are read both by rows and
// transposed: both take the 19-slot stride at D = 128 (13 at D = 64).
template <typename T, int D>
struct DkvLayout {
  static constexpr int KRB = D * (int)sizeof(T);
  static constexpr int SK = D == 128 ? 19 : 13;  // Q rows
  static constexpr int SV = SK;                  // dO rows
  static constexpr int K_BYTES = kBN * SK * 16;
  static constexpr int V_BYTES = kBN * SV * 16;
  static constexpr int K_INS = kBN * SK / kWave;
  static constexpr int V_INS = kBN * SV / kWave;
  static constexpr int V_OFF = kStages * K_BYTES;
  static constexpr int S_OFF = kStages * (K_BYTES + V_BYTES);  // L, Dl of each stage
  static constexpr int S_BYTES = 2 * kBN * 4;
  static constexpr int LDS_BYTES = S_OFF + kStages * S_BYTES;
  static constexpr uint32_t K_TILE_GLOBAL = kBN * KRB;
  static constexpr uint32_t V_TILE_GLOBAL = kBN * KRB;
  static_assert(LDS_BYTES + kWave * 16 <= 160 * 1024, "LDS");
};

// One item: the 128 keys at it.q0 (the tile's first key) of slice it.bh,
// query tiles (64 rows) [it.kt0, it.kt1).  it.slot < 0: the whole tile,
// stores dK (times scale) and dV in OT; else fp32 partial sums of dK^T and
// dV^T to workspace slot it.slot (128 keys of D each, dK then dV).
//
// MASKED: the local-window + global-token rule mk; the item's query tiles
// are the list ql (entries [kt0, kt1) are list indices, query_list), blocks
// with no visible pair are skipped, and every score is tested against the
// rule through the interval of queries that see the lane's key.
template <typename T, typename OT, int D, bool CAUSAL, bool MASKED = false>
__device__ __forceinline__ void dkv8_run(const T *__restrict__ q, const T *__restrict__ k,
                                         const T *__restrict__ v, const T *__restrict__ dout,
                                         const float *__restrict__ lse,
                                         const float *__restrict__ dl, OT *__restrict__ dk,
                                         OT *__restrict__ dv, float *__restrict__ ws, int Nq,
                                         int Nk, float c, float scale, const PipeItem it,
                                         bool reuse, const Mask mk = Mask{},
                                         const KeyList ql = KeyList{}) {
  typedef DkvLayout<T, D> L;
  typedef Dma8<T, D, T, L> DM;
  typedef typename Mma<T>::frag frag;
  constexpr int QF = D / 16;   // MFMAs of S and of dP per 32-query block
  constexpr int NDB = D / 32;  // dK^T, dV^T blocks of 32 head-dim rows
  constexpr int KT = 128;      // keys per workgroup
  __shared__ __attribute__((aligned(16))) char ring_[DM::LDS_BYTES];
  lds_char *ring = (lds_char *)ring_;
  const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;

  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave & 3, h = wave >> 2;
  const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int kw = it.q0 + kg * 32;  // this wave's first key
  const int my_k = kw + l32;
  const uint32_t rbase = (uint32_t)(l32 * L::SK * 16 + g * 16);  // row reads (Q, dO)
  uint32_t tbase;                                                 // transposed reads
  {
    const int G = lane >> 4, s16 = lane & 15;
    const int row = 4 * (G >> 1) + (s16 >> 2);
    const int col = 16 * (G & 1) + 4 * (s16 & 3);
    tbase = (uint32_t)(row * L::SK * 16 + col * 2);
  }
  const size_t qoff = (size_t)it.bh * Nq * D;
  const size_t koff = (size_t)it.bh * Nk * D;
  const u32x4 q_rs = raw_rsrc(q + qoff, (uint32_t)Nq * D * sizeof(T));
  const u32x4 do_rs = raw_rsrc(dout + qoff, (uint32_t)Nq * D * sizeof(T));
  const u32x4 k_rs = raw_rsrc(k + koff, (uint32_t)Nk * D * sizeof(T));
  const u32x4 v_rs = raw_rsrc(v + koff, (uint32_t)Nk * D * sizeof(T));
  const u32x4 l_rs = raw_rsrc(lse + (size_t)it.bh * Nq, (uint32_t)Nq * 4u);
  const u32x4 d_rs = raw_rsrc(dl + (size_t)it.bh * Nq, (uint32_t)Nq * 4u);
  DM dm;
  dm.init(ring_addr, wave, lane);
  // the L and Dl of query tile j into stage st: 16 lanes of wave 0 each
  auto issue_stats = [&](int j, int st) {
    if (wave == 0 && lane < 16) {
      const uint32_t off = (uint32_t)(j * kBN + 4 * lane) * 4u;
      const uint32_t lb = ring_addr + L::S_OFF + st * L::S_BYTES;
      dma16(l_rs, lb, off);
      dma16(d_rs, lb + kBN * 4, off);
    }
  };
  auto issue = [&](int j, int st) {
    dm.issue(q_rs, do_rs, j, st, j, st);
    issue_stats(j, st);
  };

  const int qt0 = it.kt0;
  const int ntiles = it.kt1 - it.kt0;
  // query tile of entry v (MASKED: of the list)
  auto qt_act = [&](int v) { return MASKED ? (v < ql.n1 ? v : ql.b0 + (v - ql.n1)) : v; };

  u32x4 kraw[QF], vraw[QF];
#pragma unroll
  for (int f = 0; f < QF; ++f) {
    const uint32_t off = ((uint32_t)my_k * D + 16 * f + 8 * g) * sizeof(T);
    kraw[f] = load16_async(k_rs, off);
    vraw[f] = load16_async(v_rs, off);
  }
  issue(qt_act(qt0), 0);
  if (ntiles > 1) issue(qt_act(qt0 + 1), 1);
  frag kf[QF], vf[QF];
  f32x16 dka[NDB], dva[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dka[db] = f32x16{};
    dva[db] = f32x16{};
  }

  // even steps: tiles r and r+1 have landed, and every wave is done with
  // the stages of tiles r-2 and r-1, which tiles r+2 and r+3 now take
  auto ring_step = [&](int r) {
    ring_barrier<0>();
    if (r + 2 < ntiles) issue(qt_act(qt0 + r + 2), (r + 2) & 3);
    if (r + 3 < ntiles) issue(qt_act(qt0 + r + 3), (r + 3) & 3);
  };
  ring_step(0);
#pragma unroll
  for (int f = 0; f < QF; ++f) {
    asm volatile("" : "+v"(kraw[f]), "+v"(vraw[f]));  // read after the wait above
    kf[f] = __builtin_bit_cast(frag, kraw[f]);
    vf[f] = __builtin_bit_cast(frag, vraw[f]);
  }

  const int mk4 = my_k - 4 * g;
  // MASKED: query i = sx + 4g (sx = i0 + 8 r4 + e) sees key my_k iff
  // (unsigned)(sx - bl) <= bs, or (non-causal) sx < gq: causal, the queries
  // [my_k, my_k + window - 1], or every query from my_k on for a global key;
  // non-causal, [my_k - window + 1, my_k + window - 1], every query for a
  // global key, and the global queries [0, nglobal) for any key.
  int bl = 0, gq = 0;
  unsigned bs = 0;
  if constexpr (MASKED) {
    // CAUSAL is the rule's own (the host dispatches on mk.causal)
    const bool gk = my_k < mk.nglobal;
    if (CAUSAL) {
      bl = mk4;
      bs = gk ? 0x7fffffffu : (unsigned)(mk.window - 1);
    } else {
      bl = mk4 - (mk.window - 1);
      bs = gk ? 0xffffffffu : (unsigned)(2 * mk.window - 2);
      gq = mk.nglobal - 4 * g;
    }
  }
  // Step r: query tile qt0 + r, this wave's 32 rows (i0 .. i0 + 31).  Blocks
  // with no visible pair are skipped; every other step takes the causal test
  // (two instructions a score).  Rows past Nq need no mask: their Q, dO, L
  // and Dl read as zero, so P = 1 there and dS = 0, and both meet zero rows
  // of dO and Q in dV and dK.
  auto step = [&](int r) {
    if (r > 0 && (r & 1) == 0) ring_step(r);
    const int i0 = qt_act(qt0 + r) * kBN + 32 * h;  // this wave's first query of the tile
    // wave-uniform: no query of the block sees a key of this wave
    if (MASKED ? !mk.any(i0, i0 + 31, kw, kw + 31) : (CAUSAL && i0 + 31 < kw)) return;
    if (i0 >= Nq) return;
    const int st = r & 3;
    const lds_char *qp = ring + st * L::K_BYTES + h * 32 * L::SK * 16;
    const lds_char *dp_ = ring + L::V_OFF + st * L::V_BYTES + h * 32 * L::SV * 16;
    const lds_char *sp = ring + L::S_OFF + st * L::S_BYTES + h * 32 * 4;
    f32x16 sc = f32x16{}, dpv = f32x16{};
#pragma unroll
    for (int f = 0; f < QF; ++f) {
      const frag qa = *(const __attribute__((address_space(3))) frag *)(qp + rbase + f * 32);
      const frag da = *(const __attribute__((address_space(3))) frag *)(dp_ + rbase + f * 32);
      sc = Mma<T>::mma(qa, kf[f], sc);
      dpv = Mma<T>::mma(da, vf[f], dpv);
    }
    // rows of register 4 r4 + e: query i0 + 8 r4 + 4 g + e; the two 16-row
    // halves (ks) are finished one after the other to keep registers low
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float p[8], ds[8];
#pragma unroll
      for (int hr = 0; hr < 2; ++hr) {
        const int r4 = 2 * ks + hr;
        const int ib = 8 * r4 + 4 * g;
        const f32x4 lv = *(const __attribute__((address_space(3))) f32x4 *)(sp + ib * 4);
        const f32x4 dv4 =
            *(const __attribute__((address_space(3))) f32x4 *)(sp + kBN * 4 + ib * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int x = 4 * r4 + e;
          float pr = __builtin_amdgcn_exp2f(
              __builtin_fmaf(sc[x], c, -lv[e] * 1.4426950408889634f));
          // query i0 + 8 r4 + e + 4g against key my_k: the wave-uniform
          // part of the query index against a per-lane constant
          if constexpr (MASKED) {
            const int sx = i0 + 8 * r4 + e;
            if (!((unsigned)(sx - bl) <= bs || (!CAUSAL && sx < gq))) pr = 0.f;
          } else if constexpr (CAUSAL) {
            if (mk4 > i0 + 8 * r4 + e) pr = 0.f;
          }
          p[4 * hr + e] = pr;
          ds[4 * hr + e] = pr * (dpv[x] - dv4[e]);
        }
      }
      const u32x4 pw = {Mma<T>::pack2(p[0], p[1]), Mma<T>::pack2(p[2], p[3]),
                        Mma<T>::pack2(p[4], p[5]), Mma<T>::pack2(p[6], p[7])};
      const u32x4 sw = {Mma<T>::pack2(ds[0], ds[1]), Mma<T>::pack2(ds[2], ds[3]),
                        Mma<T>::pack2(ds[4], ds[5]), Mma<T>::pack2(ds[6], ds[7])};
      const frag pb = __builtin_bit_cast(frag, pw), sb = __builtin_bit_cast(frag, sw);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const lds_char *a0 = dp_ + tbase + ks * 16 * L::SV * 16 + db * 64;
        const u32x2 lo = read_tr16(a0), hi = read_tr16(a0 + 8 * L::SV * 16);
        const u32x4 ra = {lo[0], lo[1], hi[0], hi[1]};
        dva[db] = Mma<T>::mma(__builtin_bit_cast(frag, ra), pb, dva[db]);
        const lds_char *b0 = qp + tbase + ks * 16 * L::SK * 16 + db * 64;
        const u32x2 lo2 = read_tr16(b0), hi2 = read_tr16(b0 + 8 * L::SK * 16);
        const u32x4 rb = {lo2[0], lo2[1], hi2[0], hi2[1]};
        dka[db] = Mma<T>::mma(__builtin_bit_cast(frag, rb), sb, dka[db]);
      }
    }
  };
  // One loop: the masked steps run apart from the others (two more copies
  // of the step) made the compiler spill K and V fragments.
  for (int r = 0; r < ntiles; ++r) step(r);
  wait_vmcnt<0>();    // no DMA may outlive the ring
  ring_barrier<0>();  // every wave is done with the ring

  // the odd wave of each group hands its sums to the even one
  constexpr int NR = NDB * 4;
  lds_char *xch = ring + (uint32_t)kg * 2 * NR * kWave * 16;
  if (h == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 x = {dka[db][4 * r4], dka[db][4 * r4 + 1], dka[db][4 * r4 + 2],
                         dka[db][4 * r4 + 3]};
        const f32x4 y = {dva[db][4 * r4], dva[db][4 * r4 + 1], dva[db][4 * r4 + 2],
                         dva[db][4 * r4 + 3]};
        *(__attribute__((address_space(3))) f32x4 *)(xch + ((db * 4 + r4) * kWave + lane) * 16) = x;
        *(__attribute__((address_space(3))) f32x4 *)(xch + ((NR + db * 4 + r4) * kWave + lane) * 16) = y;
      }
  }
  ring_barrier<0>();
  if (h == 0) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 x = *(const __attribute__((address_space(3))) f32x4 *)(
            xch + ((db * 4 + r4) * kWave + lane) * 16);
        const f32x4 y = *(const __attribute__((address_space(3))) f32x4 *)(
            xch + ((NR + db * 4 + r4) * kWave + lane) * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dka[db][4 * r4 + e] += x[e];
          dva[db][4 * r4 + e] += y[e];
        }
      }
    if (it.slot < 0) {
      if (my_k < Nk) {
        store_row<OT, NDB>(dka, scale, dk + ((size_t)it.bh * Nk + my_k) * D, g, D);
        store_row<OT, NDB>(dva, 1.f, dv + ((size_t)it.bh * Nk + my_k) * D, g, D);
      }
    } else {
      float *w = ws + (size_t)it.slot * 2 * KT * D;
      store_row<float, NDB>(dka, 1.f, w + (size_t)(my_k - it.q0) * D, g, D);
      store_row<float, NDB>(dva, 1.f, w + (size_t)(KT + my_k - it.q0) * D, g, D);
    }
  }
  if (reuse) ring_barrier<63, 0>();
}

// One workgroup per 128-key tile, lowest keys (the most queries) first
// under the causal mask.
// Query tiles (64 rows) that see some key of [k0, k1] under the window rule
// mk, as a list like key_list's: query tiles [0, n1), then from b0 on.
// Causal: the queries from k0 to k1 + window - 1, or to the end when the
// tile holds a global key.  Non-causal: every query for a global key;
// otherwise the global queries [0, nglobal) and the band [k0 - window + 1,
// k1 + window - 1].  *n is the list's length (0: no query sees the keys).
__device__ __forceinline__ KeyList query_list(const Mask &mk, int k0, int k1, int Nq, int *n) {
  const int nqt = (Nq + kBN - 1) / kBN;
  if (k0 < mk.nglobal) {  // a global key: every query from k0 on (causal) or every query
    const int qa = mk.causal ? min(k0 / kBN, nqt) : 0;
    *n = nqt - qa;
    return {0, qa};
  }
  const int n1 = mk.causal ? 0 : (min(mk.nglobal, Nq) + kBN - 1) / kBN;
  const int blo = mk.causal ? k0 : max(0, k0 - mk.window + 1);
  const int bhi = min(Nq - 1, k1 + mk.window - 1);
  if (blo > bhi) {  // no band query
    *n = n1;
    return {n1, n1};
  }
  const int b0 = blo / kBN, b1 = bhi / kBN + 1;
  if (b0 <= n1) {  // the ranges meet: one range from tile 0
    *n = max(n1, b1);
    return {*n, *n};
  }
  *n = n1 + (b1 - b0);
  return {n1, b0};
}

// One workgroup per 128-key tile, lowest keys (the most queries) first
// under the causal mask.  MASKED: the tile walks its query_list; with
// S > 1 the key tiles [0, nsp) (those that hold global keys, whose lists
// run over nearly every query tile) come first, each as S workgroups that
// take consecutive parts of its list and store fp32 partial sums to
// workspace slot (bh * nsp + t) * S + p (fa_merge_dkv8_split adds them).
template <typename T, typename OT, int D, bool CAUSAL, bool MASKED = false>
__global__ __launch_bounds__(kThreads8) void fa_bwd_dkdv8(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ dl,
    OT *__restrict__ dk, OT *__restrict__ dv, float *__restrict__ ws, int Nq, int Nk, int BH,
    int nkt, float c, float scale, Mask mk, int nsp, int S) {
  FA_DBG_BEGIN();
  const int id = blockIdx.x;
  const int bh = id % BH, u = id / BH;  // causal: u ascending = longest first
  int t = u, p = -1;                    // key tile, and its part (split tiles)
  if (u < nsp * S) {
    t = u / S;
    p = u % S;
  } else {
    t = u - nsp * S + nsp;
  }
  const int k0 = t * 128;
  const int nq = (Nq + kBN - 1) / kBN;
  int qa = CAUSAL ? min(k0 / kBN, nq) : 0;  // first query tile with a visible key
  int qn = nq;                              // end of the query tiles
  int slot = -1;
  KeyList ql{};
  if constexpr (MASKED) {
    int n;
    ql = query_list(mk, k0, min(k0 + 127, Nk - 1), Nq, &n);
    qa = 0;
    qn = n;
    if (p >= 0) {
      qa = (int)((int64_t)p * n / S);
      qn = (int)((int64_t)(p + 1) * n / S);
      slot = (bh * nsp + t) * S + p;
    }
  }
  const PipeItem it = {bh, k0, qa, qn, slot};
  if (qa >= qn && slot >= 0) {  // an empty part: zero partial sums
    float *w = ws + (size_t)slot * 2 * 128 * D;
    for (int i = threadIdx.x; i < 2 * 128 * D; i += kThreads8) w[i] = 0.f;
    return;
  }
  if (qa >= qn) {  // no query sees these keys: zero gradients
    for (int i = threadIdx.x; i < 128 * D; i += kThreads8) {
      const int key = k0 + i / D;
      if (key < Nk) {
        dk[((size_t)bh * Nk + key) * D + i % D] = (OT)0.f;
        dv[((size_t)bh * Nk + key) * D + i % D] = (OT)0.f;
      }
    }
    return;
  }
  dkv8_run<T, OT, D, CAUSAL, MASKED>(q, k, v, dout, lse, dl, dk, dv, ws, Nq, Nk, c, scale, it,
                                     false, mk, ql);
}

// The stream-K schedule of the forward applied to key tiles: the plan's
// "query tiles" are 128-key tiles and its units the 64-row query tiles each
// one meets.  Under the causal mask key tile t meets query tiles 2t .. n-1,
// the forward's triangle read backwards (plan tile t' = nkt - 1 - t holds
// 2(t' + 1) units) when Nq = Nk is a multiple of 128, the only causal case
// the host gives this kernel.
template <typename T, typename OT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads8) void fa_bwd_dkdv8_stream(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ dl,
    OT *__restrict__ dk, OT *__restrict__ dv, float *__restrict__ ws, int Nq, int Nk, float c,
    float scale, StreamPlan sp, ChunkStarts cs) {
  FA_DBG_BEGIN();
  ChunkWalk cw;
  const int ch = chunk_of(blockIdx.x, sp.G);
  cw.init_at(sp, ch, cs.w[2 * ch], cs.w[2 * ch + 1]);
  PipeItem it;
  int t;
  while (cw.next(sp, CAUSAL, it, t)) {
    const int kt = CAUSAL ? sp.nqt - 1 - t : t;  // the key tile
    const int base = CAUSAL ? 2 * kt : 0;          // its first query tile
    it.q0 = kt * 128;
    it.kt0 += base;
    it.kt1 += base;
    dkv8_run<T, OT, D, CAUSAL>(q, k, v, dout, lse, dl, dk, dv, ws, Nq, Nk, c, scale, it, true);
  }
}

// Sums the partial dK^T and dV^T of np pieces of key tile kt (piece kk in
// workspace slot slot_of(kk), in piece order), rows of part part of the
// tile, and stores scale times the dK sum and the dV sum.
template <typename OT, int D, typename F>
__device__ __forceinline__ void merge_dkv_rows(const float *__restrict__ ws,
                                               OT *__restrict__ dk, OT *__restrict__ dv,
                                               int Nk, float scale, int bh, int kt, int np,
                                               int part, F slot_of) {
  constexpr int C4 = D / 4;
  constexpr int RPP = kThreads / C4;
  constexpr int ROWS = merge_rows<D>();
  constexpr int NR = ROWS / RPP;
  static_assert(NR >= 1 && ROWS % RPP == 0, "merge tiling");
  const int c4 = threadIdx.x % C4;
  const int r0 = part * ROWS + threadIdx.x / C4;
  f32x4 ak[NR], av[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) ak[i] = av[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kk = 0; kk < np; ++kk) {
    const float *w = ws + (size_t)slot_of(kk) * 2 * 128 * D;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const size_t e = (size_t)(r0 + i * RPP) * D + 4 * c4;
      ak[i] += *reinterpret_cast<const f32x4 *>(w + e);
      av[i] += *reinterpret_cast<const f32x4 *>(w + 128 * D + e);
    }
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int key = kt * 128 + r0 + i * RPP;
    if (key < Nk) {
      store4<OT>(dk + ((size_t)bh * Nk + key) * D + 4 * c4, ak[i] * scale);
      store4<OT>(dv + ((size_t)bh * Nk + key) * D + 4 * c4, av[i]);
    }
  }
}

// The cut key tiles of the stream schedule (fa_bwd_dkdv8_stream).
template <typename OT, int D>
__global__ __launch_bounds__(kThreads) void fa_merge_dkv8(const float *__restrict__ ws,
                                                          OT *__restrict__ dk,
                                                          OT *__restrict__ dv, int Nk,
                                                          float scale, int nkt, bool causal,
                                                          CutList cuts) {
  constexpr int SPLIT = 128 / merge_rows<D>();
  const uint32_t w0 = cuts.w[2 * (blockIdx.x / SPLIT)];
  const uint32_t w1 = cuts.w[2 * (blockIdx.x / SPLIT) + 1];
  const int bh = (int)(w0 & 0xffffu), tp = (int)(w0 >> 16);
  const int kt = causal ? nkt - 1 - tp : tp;
  merge_dkv_rows<OT, D>(ws, dk, dv, Nk, scale, bh, kt, cut_pieces(w1), blockIdx.x % SPLIT,
                        [&](int kk) { return cut_slot(w1, kk); });
}

// The split key tiles of the masked grid (fa_bwd_dkdv8 with S > 1): tiles
// [0, nsp) of every slice, S parts each.
template <typename OT, int D>
__global__ __launch_bounds__(kThreads) void fa_merge_dkv8_split(const float *__restrict__ ws,
                                                                OT *__restrict__ dk,
                                                                OT *__restrict__ dv, int Nk,
                                                                float scale, int BH, int nsp,
                                                                int S) {
  constexpr int SPLIT = 128 / merge_rows<D>();
  const int c = blockIdx.x / SPLIT;
  const int bh = c % BH, kt = c / BH;
  const int base = (bh * nsp + kt) * S;
  merge_dkv_rows<OT, D>(ws, dk, dv, Nk, scale, bh, kt, S, blockIdx.x % SPLIT,
                        [&](int kk) { return base + kk; });
}

// The split tiles of the masked dQ grid (fa_bwd_dq8 with S > 1): tiles
// [0, nsp) of every slice, S parts each, added in part order.
template <typename OT, int D>
__global__ __launch_bounds__(kThreads) void fa_merge_dq8_split(const float *__restrict__ ws,
                                                               OT *__restrict__ dq, int Nq,
                                                               float scale, int BH, int nsp,
                                                               int S) {
  constexpr int C4 = D / 4;
  constexpr int RPP = kThreads / C4;
  constexpr int ROWS = merge_rows<D>();
  constexpr int SPLIT = 128 / ROWS;
  constexpr int NR = ROWS / RPP;
  static_assert(NR >= 1 && ROWS % RPP == 0, "merge tiling");
  const int c = blockIdx.x / SPLIT;
  const int bh = c % BH, t = c / BH;
  const size_t base = (size_t)(bh * nsp + t) * S;
  const int c4 = threadIdx.x % C4;
  const int r0 = (blockIdx.x % SPLIT) * ROWS + threadIdx.x / C4;
  f32x4 acc[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kk = 0; kk < S; ++kk) {
#pragma unroll
    for (int i = 0; i < NR; ++i)
      acc[i] += *reinterpret_cast<const f32x4 *>(
          ws + ((base + kk) * 128 + r0 + i * RPP) * D + 4 * c4);
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int row = t * 128 + r0 + i * RPP;
    if (row < Nq) store4<OT>(dq + ((size_t)bh * Nq + row) * D + 4 * c4, acc[i] * scale);
  }
}

// ---------------------------------------------------------------------------
// Stream-K schedule for variable-length batches (the dense schedule's
// balance, for packed sequences of any lengths).  The units are those of the
// dense schedule, laid out (head, sequence) pair by pair (p = h * S + s),
// each pair's query tiles in zigzag order with `lead` empty units before
// each tile; chunk c of G' = min(G, T) holds units [c T / G', (c+1) T / G').
// The offsets are in device memory, so every workgroup derives the plan
// itself at its start: the units of each pair (from the offsets), their
// prefix sums (in LDS), and by binary search where its chunk starts.  The
// workgroup of chunk j also records whether boundary j cuts a tile (as
// CutTile) in entry j of the workspace's cut table, which the combining
// kernel reads; every entry is written by every call.
constexpr int kVPairs = 512;  // (head, sequence) pairs: one per thread of the workgroup

// Rows, keys and tiles of pair p (offsets clamped to [0, T]: any offsets
// stay inside the tensors).
struct VPair {
  int h, s, qa, ka, nq, nk, ntiles, nkt;
};
__device__ __forceinline__ VPair vpair(const int *cu_q, const int *cu_k, int S, int Tq, int Tk,
                                       int p, int QT) {
  VPair r;
  r.h = p / S;
  r.s = p % S;
  r.qa = max(0, min(cu_q[r.s], Tq));
  const int qb = max(r.qa, min(cu_q[r.s + 1], Tq));
  r.ka = max(0, min(cu_k[r.s], Tk));
  const int kb = max(r.ka, min(cu_k[r.s + 1], Tk));
  r.nq = qb - r.qa;
  r.nk = kb - r.ka;
  r.ntiles = (r.nq + QT - 1) / QT;
  r.nkt = (r.nk + kBN - 1) / kBN;
  return r;
}
__device__ __forceinline__ long long vpair_units(const VPair &v, int tu, int lead, bool causal) {
  if (v.nq == 0 || v.nk == 0) return 0;
  return prefix_nat(v.ntiles, v.nkt, tu, causal) + (long long)lead * v.ntiles;
}

template <typename T, typename OT, int D, bool CAUSAL, bool PAIR>
__global__ __launch_bounds__(kThreads8) void fa_fwd_stream_varlen(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    OT *__restrict__ o, float *__restrict__ lse, float *__restrict__ ws,
    const int *__restrict__ cu_q, const int *__restrict__ cu_k, int S, int H, int Tq, int Tk,
    float c, int negate, uint32_t *__restrict__ cuts, int G) {
  FA_DBG_BEGIN();
  constexpr int QT = QRows<PAIR>::value;
  constexpr int tu = QT / kBN;
  constexpr int LEAD = varlen_lead(D, PAIR);
  static_assert(kThreads8 >= kVPairs, "one pair per thread");
  __shared__ long long pre[kVPairs + 1];
  const int NP = H * S;
  const int tid = threadIdx.x;
  // units of each pair, then their inclusive prefix sums
  if (tid < NP) {
    const VPair vp = vpair(cu_q, cu_k, S, Tq, Tk, tid, QT);
    pre[tid + 1] = vpair_units(vp, tu, LEAD, CAUSAL);
  }
  if (tid == 0) pre[0] = 0;
  __syncthreads();
  for (int off = 1; off < NP; off <<= 1) {
    const long long x = (tid < NP && tid >= off) ? pre[tid + 1 - off] : 0;
    __syncthreads();
    if (tid < NP) pre[tid + 1] += x;
    __syncthreads();
  }
  const long long TT = pre[NP];
  const int Ge = (int)(TT < G ? TT : G);
  // sequences with queries and no keys (no units): O = 0, L = -inf, their
  // pairs dealt to the workgroups
  for (int p = blockIdx.x; p < NP; p += G) {
    if (pre[p + 1] != pre[p]) continue;
    const VPair vp = vpair(cu_q, cu_k, S, Tq, Tk, p, QT);
    if (vp.nq == 0 || vp.nk != 0) continue;
    const size_t r0 = (size_t)vp.h * Tq + vp.qa;
    for (int i = tid; i < vp.nq * D; i += kThreads8) o[r0 * D + i] = (OT)0.f;
    for (int i = tid; i < vp.nq; i += kThreads8) lse[r0 + i] = -INFINITY;
  }
  if ((int)blockIdx.x >= Ge) {  // workgroup-uniform, before any barrier below
    if (tid == 0) cuts[3 * blockIdx.x + 2] = 0;  // boundary blockIdx.x: no cut
    return;
  }
  const long long cq = TT / Ge;
  const int cr = (int)(TT - cq * Ge);
  // floor(c T / G'): c r < G'^2 <= 2^16
  auto bnd = [&](int cc) { return (long long)cc * cq + (cc * cr) / Ge; };
  // the pair holding unit b: the last p with pre[p] <= b (pairs without
  // units have pre[p] = pre[p + 1] and are passed over)
  auto find = [&](long long b) {
    int lo = 0, hi = NP - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= b) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  const int ch = chunk_of(blockIdx.x, Ge);
  const long long b0 = bnd(ch);
  int p = find(b0);
  VPair vp = vpair(cu_q, cu_k, S, Tq, Tk, p, QT);
  const int zo0 = zz_find(b0 - pre[p], vp.ntiles, vp.nkt, tu, LEAD, CAUSAL);
  const long long sl0 = pre[p] + zz_prefix(zo0, vp.ntiles, vp.nkt, tu, LEAD, CAUSAL);
  int zo = zo0, u = (int)(b0 - sl0);
  // boundary ch: does it cut the tile holding it (strictly inside its key
  // tiles, the previous boundary at or before them)?
  if (tid == 0) {
    uint32_t w1 = 0, tt = 0;
    if (ch >= 1) {
      const int t = zz_tile(zo0, vp.ntiles);
      const long long s0 = sl0 + LEAD, s1 = s0 + tile_w(t, vp.nkt, tu, CAUSAL);
      const long long bp = bnd(ch - 1);
      if (b0 > s0 && b0 < s1 && bp <= s0) {
        int pieces = 1;
        for (int cc = ch; cc < Ge && bnd(cc) < s1; ++cc) ++pieces;
        // chunk ch-1 holds key tiles of an earlier tile: this is its last piece
        w1 = (uint32_t)ch | ((uint32_t)pieces << 16) | (bp < sl0 ? 1u << 31 : 0u);
        tt = (uint32_t)t;
      }
    }
    cuts[3 * ch] = (uint32_t)p;
    cuts[3 * ch + 1] = tt;
    cuts[3 * ch + 2] = w1;
  }
  long long left = bnd(ch + 1) - b0;
  bool first = true;
  while (left > 0 && p < NP) {
    if (vp.nq == 0 || vp.nk == 0) {  // a pair without units
      vp = vpair(cu_q, cu_k, S, Tq, Tk, ++p < NP ? p : NP - 1, QT);
      zo = 0;
      continue;
    }
    const int t = zz_tile(zo, vp.ntiles);
    const int w = tile_w(t, vp.nkt, tu, CAUSAL);
    const int span = LEAD + w;
    const int u1 = left < (long long)(span - u) ? u + (int)left : span;
    const int kt0 = u <= LEAD ? 0 : (u - LEAD < w ? u - LEAD : w);
    const int kt1 = u1 <= LEAD ? 0 : (u1 - LEAD < w ? u1 - LEAD : w);
    left -= u1 - u;
    u = 0;
    const VPair cur = vp;
    if (++zo == vp.ntiles) {
      zo = 0;
      if (++p < NP) vp = vpair(cu_q, cu_k, S, Tq, Tk, p, QT);
    }
    if (kt1 > kt0) {
      PipeItem it = {0, t * QT, kt0, kt1, (kt0 == 0 && kt1 == w) ? -1 : 2 * ch + (first ? 0 : 1)};
      first = false;
      const size_t qo = (size_t)cur.h * Tq + cur.qa, ko = (size_t)cur.h * Tk + cur.ka;
      pipe8_run<T, OT, D, CAUSAL, PAIR>(q + qo * D, k + ko * D, v + ko * D, o + qo * D,
                                        lse + qo, ws, cur.nq, cur.nk, c, negate, it, 2 * G);
    }
  }
}

// Combines the pieces of the varlen stream schedule's cut tiles, as
// fa_merge_stream: the workgroups of boundary j read entry j of the cut
// table (written by the stream kernel) and stop unless it names a cut.
template <typename OT, int D, int QT>
__global__ __launch_bounds__(kThreads) void fa_merge_stream_varlen(
    const float *__restrict__ ws, OT *__restrict__ o, float *__restrict__ lse,
    const int *__restrict__ cu_q, const int *__restrict__ cu_k, int S, int Tq, int Tk,
    const uint32_t *__restrict__ cuts, int G) {
  constexpr int C4 = D / 4;
  constexpr int RPP = kThreads / C4;
  constexpr int SPLIT = QT / merge_rows<D>();
  constexpr int ROWS = merge_rows<D>();
  constexpr int NR = ROWS / RPP;
  static_assert(NR >= 1 && ROWS % RPP == 0, "merge tiling");
  const uint32_t *cut = cuts + 3 * (1 + blockIdx.x / SPLIT);  // boundary 1 + blockIdx / SPLIT
  const uint32_t w1 = cut[2];
  if (w1 == 0) return;  // not a cut
  const int p = (int)cut[0], t = (int)cut[1];
  const int np = cut_pieces(w1);
  const VPair vp = vpair(cu_q, cu_k, S, Tq, Tk, p, QT);
  const int rbase = (blockIdx.x % SPLIT) * ROWS;
  const int c4 = threadIdx.x % C4;
  const int r0 = rbase + threadIdx.x / C4;
  const float *ws_s = ws + (size_t)2 * G * QT * D;
  float M[NR], ls[NR], lrs[NR];
  f32x4 acc[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    M[i] = -INFINITY;
    ls[i] = lrs[i] = 0.f;
    acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int kk = 0; kk < np; kk += 2) {
    const int sl[2] = {cut_slot(w1, kk), kk + 1 < np ? cut_slot(w1, kk + 1) : -1};
    f32x4 st[2][NR], x[2][NR];
#pragma unroll
    for (int uu = 0; uu < 2; ++uu)
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        if (sl[uu] < 0) continue;
        const size_t e = (size_t)sl[uu] * QT + r0 + i * RPP;
        st[uu][i] = *reinterpret_cast<const f32x4 *>(ws_s + e * 4);
        x[uu][i] = *reinterpret_cast<const f32x4 *>(ws + e * D + 4 * c4);
      }
#pragma unroll
    for (int uu = 0; uu < 2; ++uu)
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        if (sl[uu] < 0 || st[uu][i][0] == -INFINITY) continue;  // no key of this row
        const float Mn = fmaxf(M[i], st[uu][i][0]);
        const float a_old = exp2f(M[i] - Mn);  // 0 while M = -inf
        const float a = exp2f(st[uu][i][0] - Mn);
        ls[i] = ls[i] * a_old + a * st[uu][i][1];
        lrs[i] = lrs[i] * a_old + a * st[uu][i][2];
        acc[i] = acc[i] * a_old + (a * st[uu][i][2]) * x[uu][i];
        M[i] = Mn;
      }
  }
  const size_t base = (size_t)vp.h * Tq + vp.qa + (size_t)t * QT;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int r = r0 + i * RPP;
    if (t * QT + r < vp.nq) {
      store4<OT>(o + (base + r) * D + 4 * c4, acc[i] * (1.0f / lrs[i]));
      if (c4 == 0) lse[base + r] = (M[i] + log2f(ls[i])) * 0.69314718055994531f;
    }
  }
}


template <typename T, typename OT, int D, bool CAUSAL, bool PAIR, typename KT = T>
__global__ __launch_bounds__(kThreads8) void fa_fwd_stream(
    const KT *__restrict__ q, const KT *__restrict__ k, const T *__restrict__ v,
    OT *__restrict__ o, float *__restrict__ lse, float *__restrict__ ws, int Nq, int Nk,
    float c, int negate, StreamPlan sp, ChunkStarts cs, float osc) {
  FA_DBG_BEGIN();
  ChunkWalk cw;
  const int ch = chunk_of(blockIdx.x, sp.G);
  cw.init_at(sp, ch, cs.w[2 * ch], cs.w[2 * ch + 1]);
  PipeItem it;
  int t;
  while (cw.next(sp, CAUSAL, it, t)) {
    it.q0 = t * QRows<PAIR>::value;
    pipe8_run<T, OT, D, CAUSAL, PAIR, false, KT>(q, k, v, o, lse, ws, Nq, Nk, c, negate, it,
                                                 2 * sp.G, Mask{}, KeyList{}, osc);
  }
}

// Combines the pieces of the cut query tiles (CutList), one workgroup per
// merge_rows<D>() rows of a tile, with a_i = 2^(m_i - M), M = max_i m_i:
// O = sum_i a_i lr_i O_i / sum_i a_i lr_i, L = ln2 * (M + log2 sum_i a_i l_i).
// Each thread owns one 4-wide column slice of NR rows and loads two pieces
// per round trip.

template <typename OT, int D, bool CAUSAL, int QT>
__global__ __launch_bounds__(kThreads) void fa_merge_stream(const float *__restrict__ ws,
                                                            OT *__restrict__ o,
                                                            float *__restrict__ lse, int Nq,
                                                            StreamPlan sp, CutList cuts) {
  constexpr int C4 = D / 4;           // float4 per row
  constexpr int RPP = kThreads / C4;  // rows per pass of the workgroup
  constexpr int SPLIT = QT / merge_rows<D>();
  constexpr int ROWS = merge_rows<D>();
  constexpr int NR = ROWS / RPP;      // rows per thread
  static_assert(NR >= 1 && ROWS % RPP == 0, "merge tiling");
  const uint32_t w0 = cuts.w[2 * (blockIdx.x / SPLIT)];
  const uint32_t w1 = cuts.w[2 * (blockIdx.x / SPLIT) + 1];
  const int bh = (int)(w0 & 0xffffu), t = (int)(w0 >> 16);
  const int np = cut_pieces(w1);
  const int rbase = (blockIdx.x % SPLIT) * ROWS;
  const int c4 = threadIdx.x % C4;
  const int r0 = rbase + threadIdx.x / C4;
  const int nslots = 2 * sp.G;
  const float *ws_s = ws + (size_t)nslots * QT * D;
  float M[NR], ls[NR], lrs[NR];
  f32x4 acc[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    M[i] = -INFINITY;
    ls[i] = lrs[i] = 0.f;
    acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int k = 0; k < np; k += 2) {
    const int sl[2] = {cut_slot(w1, k), k + 1 < np ? cut_slot(w1, k + 1) : -1};
    f32x4 st[2][NR], x[2][NR];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        if (sl[u] < 0) continue;
        const size_t e = (size_t)sl[u] * QT + r0 + i * RPP;
        st[u][i] = *reinterpret_cast<const f32x4 *>(ws_s + e * 4);
        x[u][i] = *reinterpret_cast<const f32x4 *>(ws + e * D + 4 * c4);
      }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        if (sl[u] < 0 || st[u][i][0] == -INFINITY) continue;  // no key of this row
        const float Mn = fmaxf(M[i], st[u][i][0]);
        const float a_old = exp2f(M[i] - Mn);  // 0 while M = -inf
        const float a = exp2f(st[u][i][0] - Mn);
        ls[i] = ls[i] * a_old + a * st[u][i][1];
        lrs[i] = lrs[i] * a_old + a * st[u][i][2];
        acc[i] = acc[i] * a_old + (a * st[u][i][2]) * x[u][i];
        M[i] = Mn;
      }
    if (sl[1] < 0) break;
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int row = t * QT + r0 + i * RPP;
    if (row < Nq) {
      store4<OT>(o + ((size_t)bh * Nq + row) * D + 4 * c4, acc[i] * (1.0f / lrs[i]));
      if (c4 == 0) lse[(size_t)bh * Nq + row] = (M[i] + log2f(ls[i])) * 0.69314718055994531f;
    }
  }
}

// Combines the key chunks of the split tiles of fa_fwd_varlen, one workgroup
// per merge_rows<D>() rows of every (tile rank, head, sequence); tiles that
// were not split (or lie past their sequence's end) return at once.  Same
// rescaling as fa_merge_stream.
// Combines the partial results of np parts of one tile (part u in slot
// slot_of(u): the normalised O_p at ws, the record (m, l, lr, 0) at ws_s, as
// epilogue_partial writes them) for the rows of part `part` of the tile
// (merge_rows<D>() rows each), and stores O and L of the tile's rows below
// nrows at o_tile and lse_tile.  A row that no part saw stores O = 0 and
// L = -inf.
template <typename OT, int D, int QT, typename F>
__device__ __forceinline__ void merge_part_rows(const float *__restrict__ ws,
                                                const float *__restrict__ ws_s, int np,
                                                int part, F slot_of, OT *__restrict__ o_tile,
                                                float *__restrict__ lse_tile, int nrows) {
  constexpr int C4 = D / 4;
  constexpr int RPP = kThreads / C4;
  constexpr int ROWS = merge_rows<D>();
  constexpr int NR = ROWS / RPP;
  static_assert(NR >= 1 && ROWS % RPP == 0, "merge tiling");
  const int c4 = threadIdx.x % C4;
  const int r0 = part * ROWS + threadIdx.x / C4;
  float M[NR], ls[NR], lrs[NR];
  f32x4 acc[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    M[i] = -INFINITY;
    ls[i] = lrs[i] = 0.f;
    acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // four parts per round trip: their loads are issued before any is used
  constexpr int U = 4;
  for (int ch = 0; ch < np; ch += U) {
    f32x4 st[U][NR], x[U][NR];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ch + u >= np) break;
      const size_t slot = (size_t)slot_of(ch + u);
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const size_t e = slot * QT + r0 + i * RPP;
        st[u][i] = *reinterpret_cast<const f32x4 *>(ws_s + e * 4);
        x[u][i] = *reinterpret_cast<const f32x4 *>(ws + e * D + 4 * c4);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ch + u >= np) break;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        if (st[u][i][0] == -INFINITY) continue;  // no key of this row in the part
        const float Mn = fmaxf(M[i], st[u][i][0]);
        const float a_old = exp2f(M[i] - Mn);  // 0 while M = -inf
        const float a = exp2f(st[u][i][0] - Mn);
        ls[i] = ls[i] * a_old + a * st[u][i][1];
        lrs[i] = lrs[i] * a_old + a * st[u][i][2];
        acc[i] = acc[i] * a_old + (a * st[u][i][2]) * x[u][i];
        M[i] = Mn;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int r = r0 + i * RPP;
    if (r < nrows) {
      const float inv = lrs[i] > 0.f ? 1.0f / lrs[i] : 0.f;
      store4<OT>(o_tile + (size_t)r * D + 4 * c4, acc[i] * inv);
      if (c4 == 0)
        lse_tile[r] = lrs[i] > 0.f ? (M[i] + log2f(ls[i])) * 0.69314718055994531f : -INFINITY;
    }
  }
}

// The split tiles of the masked grid (fa_fwd_pipe8 with S > 1): tiles
// [0, nsp) of every slice, S parts each.
template <typename OT, int D, int QT>
__global__ __launch_bounds__(kThreads) void fa_merge_masked_split(
    const float *__restrict__ ws, OT *__restrict__ o, float *__restrict__ lse, int Nq, int BH,
    int nsp, int S) {
  constexpr int SPLIT = QT / merge_rows<D>();
  const int c = blockIdx.x / SPLIT;
  const int bh = c % BH, t = c / BH;
  const int base = (bh * nsp + t) * S;
  const size_t r0 = (size_t)bh * Nq + (size_t)t * QT;
  merge_part_rows<OT, D, QT>(ws, ws + (size_t)BH * nsp * S * QT * D, S, blockIdx.x % SPLIT,
                             [&](int u) { return base + u; }, o + r0 * D, lse + r0,
                             min(QT, Nq - t * QT));
}

template <typename OT, int D, bool CAUSAL, int QT>
__global__ __launch_bounds__(kThreads) void fa_merge_varlen(
    const float *__restrict__ ws, OT *__restrict__ o, float *__restrict__ lse,
    const int *__restrict__ cu_q, const int *__restrict__ cu_k, int S, int H, int Tq,
    int Tk, int NC, int KC, int NT) {
  constexpr int SPLIT = QT / merge_rows<D>();
  const int id = blockIdx.x / SPLIT;
  const int qt = id / (H * S), hs = id % (H * S);
  const int h = hs / S, sq = hs % S;
  const int qa = max(0, min(cu_q[sq], Tq)), qb = max(qa, min(cu_q[sq + 1], Tq));
  const int ka = max(0, min(cu_k[sq], Tk)), kb = max(ka, min(cu_k[sq + 1], Tk));
  const int nq = qb - qa, nk = kb - ka;
  const int q0 = qt * QT;
  if (q0 >= nq || nk == 0) return;
  const int kend = CAUSAL ? min(nk, q0 + QT) : nk;
  const int nkt = (kend + kBN - 1) / kBN;
  int kc;
  const int nch = varlen_split(nkt, NC, KC, kc);
  if (nch <= 1) return;  // written by its only workgroup
  const int nslots = H * NT * NC;
  const size_t base = (size_t)h * Tq + qa + q0;
  merge_part_rows<OT, D, QT>(ws, ws + (size_t)nslots * QT * D, nch, blockIdx.x % SPLIT,
                             [&](int ch) { return varlen_slot(h, NT, NC, qa, q0, QT, sq, ch); },
                             o + base * D, lse + base, nq - q0);
}

// ---------------------------------------------------------------------------
// fp32 inputs: same structure on v_mfma_f32_32x32x2_f32 (true fp32 products).
//
// Key split (the sequence parallelism of page "FlashAttention技术演进全景图"
// §3.2): with nsplit > 1, workgroup id handles query tile item id / nsplit
// (longest first, as work_item) and its key tiles [c KC, (c+1) KC),
// c = id % nsplit.  A tile whose keys fit one chunk is stored directly; the
// chunks of a longer tile write partials (epilogue_partial) to slot id of
// ws, which fa_merge_split32 combines.  A fp32 MFMA takes 64 cycles for its
// 4096 flops, so one 32-row wave needs about 3.4 us per 64-key tile: without
// the split, shapes with few query tiles leave most SIMDs idle while each
// wave walks every key.
__device__ __forceinline__ int split32_chunks(int q0, int Nk, int KC, bool causal) {
  const int kend = causal ? min(Nk, q0 + kBM) : Nk;
  const int nkt = (kend + kBN - 1) / kBN;
  return (nkt + KC - 1) / KC;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fa_fwd_f32(
    const float *__restrict__ q, const float *__restrict__ k,
    const float *__restrict__ v, float *__restrict__ o, float *__restrict__ lse,
    int Nq, int Nk, int BH, int nqt, float c, int KC, int nsplit, float *__restrict__ ws) {
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

  const int item = blockIdx.x / nsplit, chunk = blockIdx.x % nsplit;
  const WorkItem wi = {item % BH, (CAUSAL ? nqt - 1 - item / BH : item / BH) * kBM};
  const int nch = nsplit > 1 ? split32_chunks(wi.q0, Nk, KC, CAUSAL) : 1;
  if (chunk >= nch) return;  // a short causal tile needs fewer chunks
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
  const int kt0 = nch > 1 ? chunk * KC : 0;
  const int nkt = nch > 1 ? min((kend + kBN - 1) / kBN, kt0 + KC) : (kend + kBN - 1) / kBN;

  gload(kt0);
  swrite(0);
  __syncthreads();

  for (int kt = kt0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) gload(kt + 1);
    const int k0 = kt * kBN;
    const bool active = !CAUSAL || (k0 <= qw + 31);
    if (active) {
      const float *Ks = smem + ((kt - kt0) & 1) * BUF;
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
    if (kt + 1 < nkt) swrite((kt + 1 - kt0) & 1);
    __syncthreads();
  }

  if (nch == 1) {
    epilogue<D, float>(acc, m, l, o, lse, wi.bh, Nq, my_q, g);
  } else {
    const int nslots = BH * nqt * nsplit;
    const int row = my_q - wi.q0;
    epilogue_partial<D>(acc, m, l, l + __shfl_xor(l, 32), ws + (size_t)blockIdx.x * kBM * D,
                        ws + (size_t)nslots * kBM * D + (size_t)blockIdx.x * kBM * 4, row, g);
  }
}

// Combines the key chunks of the fp32 kernel's split tiles (slots item *
// nsplit + c), merge_rows<D>() rows per workgroup, with the rescaling of
// fa_merge_varlen; tiles left whole return at once.
template <int D>
__global__ __launch_bounds__(kThreads) void fa_merge_split32(const float *__restrict__ ws,
                                                             float *__restrict__ o,
                                                             float *__restrict__ lse, int Nq,
                                                             int Nk, int BH, int nqt, int KC,
                                                             int nsplit, bool causal) {
  constexpr int C4 = D / 4;
  constexpr int RPP = kThreads / C4;
  constexpr int ROWS = merge_rows<D>();
  constexpr int SPLIT = kBM / ROWS;
  constexpr int NR = ROWS / RPP;
  static_assert(NR >= 1 && ROWS % RPP == 0, "merge tiling");
  const int item = blockIdx.x / SPLIT;
  const int bh = item % BH;
  const int q0 = (causal ? nqt - 1 - item / BH : item / BH) * kBM;
  const int nch = split32_chunks(q0, Nk, KC, causal);
  if (nch <= 1) return;  // stored by its only workgroup
  const int nslots = BH * nqt * nsplit;
  const float *ws_s = ws + (size_t)nslots * kBM * D;
  const int c4 = threadIdx.x % C4;
  const int r0 = (blockIdx.x % SPLIT) * ROWS + threadIdx.x / C4;
  float M[NR], ls[NR], lrs[NR];
  f32x4 acc[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    M[i] = -INFINITY;
    ls[i] = lrs[i] = 0.f;
    acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  constexpr int U = 4;  // chunks per round trip
  for (int ch = 0; ch < nch; ch += U) {
    f32x4 st[U][NR], x[U][NR];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ch + u >= nch) break;
      const size_t slot = (size_t)item * nsplit + ch + u;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const size_t e = slot * kBM + r0 + i * RPP;
        st[u][i] = *reinterpret_cast<const f32x4 *>(ws_s + e * 4);
        x[u][i] = *reinterpret_cast<const f32x4 *>(ws + e * D + 4 * c4);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ch + u >= nch) break;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        if (st[u][i][0] == -INFINITY) continue;  // no key of this row in the chunk
        const float Mn = fmaxf(M[i], st[u][i][0]);
        const float a_old = exp2f(M[i] - Mn);  // 0 while M = -inf
        const float a = exp2f(st[u][i][0] - Mn);
        ls[i] = ls[i] * a_old + a * st[u][i][1];
        lrs[i] = lrs[i] * a_old + a * st[u][i][2];
        acc[i] = acc[i] * a_old + (a * st[u][i][2]) * x[u][i];
        M[i] = Mn;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int row = q0 + r0 + i * RPP;
    if (row < Nq) {
      store4<float>(o + ((size_t)bh * Nq + row) * D + 4 * c4, acc[i] * (1.0f / lrs[i]));
      if (c4 == 0) lse[(size_t)bh * Nq + row] = (M[i] + log2f(ls[i])) * 0.69314718055994531f;
    }
  }
}

// ---------------------------------------------------------------------------
// FP8 inputs on the pipelined kernel (fa_fwd_fp8_ws): Q and K stay e4m3 and
// meet on the FP8 MFMA; P.V runs on the bf16 MFMA, so V's e4m3 values are
// first widened to bf16 (exactly: e4m3's 3 fraction bits and exponent range
// fit in bf16) into the workspace by this pass, 16 values per thread.
__global__ __launch_bounds__(256) void fa_fp8_widen(const u32x4 *__restrict__ src,
                                                    u32x4 *__restrict__ dst, size_t n16) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const u32x4 w = src[i];
  uint32_t x[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w[j], false);  // bytes 0, 1
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w[j], true);   // bytes 2, 3
    x[2 * j] = Mma<__bf16>::pack2(a[0], a[1]);
    x[2 * j + 1] = Mma<__bf16>::pack2(b[0], b[1]);
  }
  dst[2 * i] = u32x4{x[0], x[1], x[2], x[3]};
  dst[2 * i + 1] = u32x4{x[4], x[5], x[6], x[7]};
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
  float *ws;
  int Nq, Nk, BH, nqt, nqtg;  // query tiles of kBM rows and of the 8-wave grid's rows
  float c;
  hipStream_t stream;
  const StreamPlan *plan;      // non-null: stream-K schedule (pipelined kernel only)
  int KC, nsplit;             // the fp32 kernel's key split (nsplit 1: none)
  float osc;                  // factor of O (FP8: the V descale; else 1)
  const ChunkStarts *starts;  // the schedule's chunk starts
  const CutList *cuts;        // the schedule's cut tiles
  bool masked;                // the window rule mk (grid path only)
  Mask mk;
  size_t ws_bytes = 0;        // masked: workspace for the split tiles' parts
};

// Split of the masked grid (the rule without causality): a 256-row tile that
// holds global queries sees every key tile, while a band tile's list holds
// the global key tiles and about (255 + 2 (window - 1)) / 64 band tiles; one
// workgroup walking a whole sequence would outlast the grid.  Those tiles
// (the first ceil(min(G, Nq) / 256) of each slice) run as S parts of about a
// band tile's list each, at least 32 key tiles; S is limited to what the
// workspace holds, and below 2 they run whole.
struct FwdSplit {
  int nsp = 0, S = 1;
};
FwdSplit fwd_masked_split(const Mask &mk, int64_t BH, int64_t Nq, int64_t Nk, int64_t D,
                          size_t avail) {
  FwdSplit r;
  const int64_t gq = mk.nglobal < Nq ? mk.nglobal : Nq;
  if (mk.causal || gq <= 0 || Nk <= 0) return r;
  constexpr int64_t QT = QRows<false>::value;
  const int64_t nkt = (Nk + kBN - 1) / kBN;
  const int64_t gk = mk.nglobal < Nk ? mk.nglobal : Nk;
  int64_t band = (gk + kBN - 1) / kBN + (QT - 1 + 2 * ((int64_t)mk.window - 1)) / kBN + 2;
  if (band > nkt) band = nkt;
  const int64_t cap = band > 32 ? band : 32;
  const int64_t nsp = (gq + QT - 1) / QT;
  const size_t per = (size_t)(BH * nsp) * QT * (size_t)(D + 4) * 4;  // one part of each
  int64_t S = (nkt + cap - 1) / cap;
  if ((size_t)S > avail / per) S = (int64_t)(avail / per);
  if (S < 2) return r;
  r.nsp = (int)nsp;
  r.S = (int)S;
  return r;
}
size_t fwd_masked_split_bytes(const FwdSplit &sp, int64_t BH, int64_t D) {
  if (sp.S < 2) return 0;
  return (size_t)(BH * sp.nsp) * sp.S * QRows<false>::value * (size_t)(D + 4) * 4;
}

template <typename T, typename OT, int D, bool CAUSAL, typename KT = T>
hipError_t launch16(const Launch &a) {
  // c > 0 here: a negative scale flips the sign of Q inside the kernel,
  // and scale 0 runs as the smallest normal scale (scores of at most
  // 2^-126 * |q.k|, which round to 0 against any shift the softmax uses).
  const float c = fmaxf(a.c < 0.f ? -a.c : a.c, 1.17549435e-38f);
  const int neg = a.c < 0.f ? 1 : 0;
  if (a.plan) {
    const StreamPlan &sp = *a.plan;
    // the plan's tile height selects the layout (pair-split: 128 rows)
    auto go = [&](auto pair) -> hipError_t {
      constexpr bool PAIR = decltype(pair)::value;
      // the workspace slots and tile indices of the plan are in units of the
      // kernel's tile height: never launch with another
      if (sp.tu * kKeys != QRows<PAIR>::value) return hipErrorInvalidValue;
      hipLaunchKernelGGL((fa_fwd_stream<T, OT, D, CAUSAL, PAIR, KT>), dim3((unsigned)sp.G),
                         dim3(kThreads8), 0, a.stream, (const KT *)a.q, (const KT *)a.k,
                         (const T *)a.v, (OT *)a.o, a.lse, a.ws, a.Nq, a.Nk, c, neg, sp,
                         *a.starts, a.osc);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (a.cuts && a.cuts->n > 0) {
        hipLaunchKernelGGL((fa_merge_stream<OT, D, CAUSAL, QRows<PAIR>::value>),
                           dim3((unsigned)(a.cuts->n * (QRows<PAIR>::value / merge_rows<D>()))),
                           dim3(kThreads), 0, a.stream, (const float *)a.ws, (OT *)a.o,
                           a.lse, a.Nq, sp, *a.cuts);
      }
      return hipSuccess;
    };
    hipError_t e;
    if constexpr (D == 128)
      e = sp.tu == kPairRows / kKeys ? go(std::true_type{}) : go(std::false_type{});
    else
      e = go(std::false_type{});
    if (e != hipSuccess) return e;
  } else if (a.masked) {
    if constexpr (std::is_same<KT, T>::value) {
      const FwdSplit sl = fwd_masked_split(a.mk, a.BH, a.Nq, a.Nk, D, a.ws ? a.ws_bytes : 0);
      const int units = a.nqtg + sl.nsp * (sl.S - 1);
      hipLaunchKernelGGL((fa_fwd_pipe8<T, OT, D, CAUSAL, false, true>),
                         dim3((unsigned)(a.BH * units)), dim3(kThreads8), 0, a.stream,
                         (const T *)a.q, (const T *)a.k, (const T *)a.v, (OT *)a.o, a.lse,
                         a.Nq, a.Nk, a.BH, a.nqtg, c, neg, a.mk, 1.f, a.ws, sl.nsp, sl.S);
      if (sl.S > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        constexpr int QT = QRows<false>::value;
        hipLaunchKernelGGL((fa_merge_masked_split<OT, D, QT>),
                           dim3((unsigned)(a.BH * sl.nsp * (QT / merge_rows<D>()))),
                           dim3(kThreads), 0, a.stream, (const float *)a.ws, (OT *)a.o, a.lse,
                           a.Nq, a.BH, sl.nsp, sl.S);
      }
    } else {
      return hipErrorInvalidValue;  // the window mask runs on 16-bit inputs only
    }
  } else {
    hipLaunchKernelGGL((fa_fwd_pipe8<T, OT, D, CAUSAL, false, false, KT>),
                       dim3((unsigned)(a.BH * a.nqtg)), dim3(kThreads8), 0, a.stream,
                       (const KT *)a.q, (const KT *)a.k, (const T *)a.v, (OT *)a.o, a.lse,
                       a.Nq, a.Nk, a.BH, a.nqtg, c, neg, Mask{}, a.osc, (float *)nullptr, 0, 1);
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch32(const Launch &a) {
  const dim3 grid((unsigned)(a.BH * a.nqt * a.nsplit)), block(kThreads);
  hipLaunchKernelGGL((fa_fwd_f32<D, CAUSAL>), grid, block, 0, a.stream,
                     (const float *)a.q, (const float *)a.k, (const float *)a.v,
                     (float *)a.o, a.lse, a.Nq, a.Nk, a.BH, a.nqt, a.c, a.KC, a.nsplit, a.ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit < 2) return e;
  hipLaunchKernelGGL((fa_merge_split32<D>),
                     dim3((unsigned)(a.BH * a.nqt * (kBM / merge_rows<D>()))), block, 0,
                     a.stream, (const float *)a.ws, (float *)a.o, a.lse, a.Nq, a.Nk, a.BH,
                     a.nqt, a.KC, a.nsplit, CAUSAL);
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

// Per-head slices are addressed with 32-bit byte offsets (plus slack past
// the end for ragged rows), and the grid is one-dimensional.  PRE: B, H,
// Nq, Nk >= 1 and D in {16, 32, 64, 128}.  No product below can overflow:
// each factor is bounded first.
bool sizes_fit(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D) {
  const int64_t lim = (int64_t)1 << 31;
  if (Nq > lim / (D * 4) - QRows<false>::value || Nk > lim / (D * 4) - 5 * kBN) return false;
  if (B > lim || H > lim || B * H > lim) return false;
  return B * H * ((Nq + kBM - 1) / kBM) < lim;
}

// Sizes of the arguments of one call, filled by validate().
struct Shape {
  int64_t BH, nqt;
  size_t qb, kb, ob, lb;
};

int validate(const void *q, const void *k, const void *v, const void *o, const float *lse,
             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, float scale,
             int dtype, Shape &sh) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULLPTR;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  if (D != 16 && D != 32 && D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  if (dtype < FA_F32 || dtype > FA_F16_OF32) return FA_ERR_DTYPE;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const int64_t in_size = (dtype == FA_F32) ? 4 : 2;
  const int64_t out_size =
      (dtype == FA_F32 || dtype == FA_BF16_OF32 || dtype == FA_F16_OF32) ? 4 : 2;
  if (!sizes_fit(B, H, Nq, Nk, D)) return FA_ERR_SHAPE;
  sh.BH = B * H;
  sh.nqt = (Nq + kBM - 1) / kBM;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGN;
  if ((uintptr_t)lse & 3u) return FA_ERR_ALIGN;
  sh.qb = (size_t)(sh.BH * Nq * D * in_size);
  sh.kb = (size_t)(sh.BH * Nk * D * in_size);
  sh.ob = (size_t)(sh.BH * Nq * D * out_size);
  sh.lb = (size_t)(sh.BH * Nq * 4);
  if (overlaps(o, sh.ob, q, sh.qb) || overlaps(o, sh.ob, k, sh.kb) ||
      overlaps(o, sh.ob, v, sh.kb) || overlaps(lse, sh.lb, q, sh.qb) ||
      overlaps(lse, sh.lb, k, sh.kb) || overlaps(lse, sh.lb, v, sh.kb) ||
      overlaps(o, sh.ob, lse, sh.lb))
    return FA_ERR_OVERLAP;
  return FA_OK;
}

// Compute units of the current device, queried once per device.
int device_cus(int *cus) {
  static int cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev >= 0 && dev < 64 && __atomic_load_n(&cache[dev], __ATOMIC_RELAXED) > 0) {
    *cus = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    return FA_OK;
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev >= 0 && dev < 64) __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
  *cus = n;
  return FA_OK;
}

// Key split of the fp32 kernel (fa_fwd_f32): used when the query tiles
// number fewer than the compute units.  The chunk length KC (64-key tiles)
// is the smallest that keeps the workgroups within one per compute unit
// (one round) and a tile within four chunks (which the combine reads in
// one round trip).  Measured on B8 N1000 D64 fp32, against chunks of 1, 2,
// 3 and 6 tiles: the 4-tile chunks this gives were fastest both causal and
// not (31.7 and 33.9 us, 2.7x and 2.5x the unsplit grid); two workgroups
// per compute unit gained nothing over one, and extra chunks per tile cost
// more in the combine than the shorter chunks saved.  The workspace is at
// most four slots of 128 rows * (D + 4) floats per compute unit.
struct Split32 {
  int KC = 0, nsplit = 1;
};

bool plan32(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, bool causal, int cus, Split32 &ks,
            size_t &bytes) {
  bytes = 0;
  ks = Split32{};
  const int64_t nqt = (Nq + kBM - 1) / kBM;
  const int64_t units = BH * nqt;
  if (cus < 1 || units >= cus) return false;
  auto keys = [&](int64_t t) {  // 64-key tiles of query tile t
    const int64_t kend = causal ? (Nk < (t + 1) * kBM ? Nk : (t + 1) * kBM) : Nk;
    return (kend + kBN - 1) / kBN;
  };
  const int64_t longest = keys(nqt - 1);  // the last tile's range is the longest
  int64_t kc = (longest + 3) / 4;
  for (;; ++kc) {
    int64_t wgs = 0;
    for (int64_t t = 0; t < nqt; ++t) wgs += (keys(t) + kc - 1) / kc;
    if (BH * wgs <= cus || kc >= longest) break;
  }
  const int64_t ns = (longest + kc - 1) / kc;
  if (ns < 2) return false;
  ks.KC = (int)kc;
  ks.nsplit = (int)ns;
  bytes = (size_t)units * (size_t)ns * kBM * (size_t)(D + 4) * 4;
  return true;
}

// The workspace a call takes, if any: the stream-K schedule of the
// pipelined kernel (16-bit inputs) or the fp32 kernel's key split.
bool plan_ws(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, int dtype, bool causal, int cus,
             StreamPlan &pl, Split32 &ks, size_t &bytes) {
  ks = Split32{};
  if (dtype == FA_F32) return plan32(BH, Nq, Nk, D, causal, cus, ks, bytes);
  return make_plan(BH, Nq, Nk, D, dtype, causal, cus, pl, bytes);
}

int run(const void *q, const void *k, const void *v, void *o, float *lse, int64_t Nq,
        int64_t Nk, int64_t D, float scale, int causal, int dtype, const Shape &sh,
        const StreamPlan *plan, void *ws, void *stream, const Mask *mk = nullptr,
        const Split32 *ks = nullptr, size_t ws_bytes = 0) {
  Launch a;
  a.ws_bytes = ws_bytes;
  a.osc = 1.f;
  a.KC = ks ? ks->KC : 0;
  a.nsplit = ks ? ks->nsplit : 1;
  a.masked = mk != nullptr;
  a.mk = mk ? *mk : Mask{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.ws = (float *)ws;
  a.Nq = (int)Nq;
  a.Nk = (int)Nk;
  a.BH = (int)sh.BH;
  a.nqt = (int)sh.nqt;
  a.nqtg = (int)((Nq + QRows<false>::value - 1) / QRows<false>::value);
  a.c = scale * 1.4426950408889634f;
  a.stream = (hipStream_t)stream;
  a.plan = plan;
  ChunkStarts starts;
  CutList cuts;
  a.starts = nullptr;
  a.cuts = nullptr;
  if (plan) {
    make_tables(*plan, causal != 0, starts, cuts);
    a.starts = &starts;
    a.cuts = &cuts;
  }
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

struct VarlenArgs {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const int *cu_q, *cu_k;
  int S, H, Tq, Tk, maxq;
  bool pair;  // pair-split 128-row tiles (D = 128 only)
  float c;
  float *ws;        // partial results of split tiles (NC > 1)
  int NC, KC, NT;   // chunks per tile at most, 64-key tiles per chunk at least, tile ids per head
  int G;            // > 0: the stream schedule with G workgroups (plan at ws + plan_off)
  size_t plan_off;
  hipStream_t stream;
};

template <typename T, typename OT, int D, bool CAUSAL>
hipError_t launch_varlen(const VarlenArgs &a) {
  // as launch16: a negative scale flips Q's sign in the kernel, scale 0 runs
  // as the smallest normal scale
  const float c = fmaxf(a.c < 0.f ? -a.c : a.c, 1.17549435e-38f);
  const int neg = a.c < 0.f ? 1 : 0;
  auto go = [&](auto pair) -> hipError_t {
    constexpr bool PAIR = decltype(pair)::value;
    constexpr int QT = QRows<PAIR>::value;
    if (a.G > 0) {
      uint32_t *cuts = (uint32_t *)((char *)a.ws + a.plan_off);
      hipLaunchKernelGGL((fa_fwd_stream_varlen<T, OT, D, CAUSAL, PAIR>), dim3((unsigned)a.G),
                         dim3(kThreads8), 0, a.stream, (const T *)a.q, (const T *)a.k,
                         (const T *)a.v, (OT *)a.o, a.lse, a.ws, a.cu_q, a.cu_k, a.S, a.H,
                         a.Tq, a.Tk, c, neg, cuts, a.G);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess || a.G < 2) return e;
      constexpr int SPLIT = QT / merge_rows<D>();
      hipLaunchKernelGGL((fa_merge_stream_varlen<OT, D, QT>),
                         dim3((unsigned)((a.G - 1) * SPLIT)), dim3(kThreads), 0, a.stream,
                         (const float *)a.ws, (OT *)a.o, a.lse, a.cu_q, a.cu_k, a.S, a.Tq,
                         a.Tk, (const uint32_t *)cuts, a.G);
      return hipGetLastError();
    }
    const int ntiles = (a.maxq + QT - 1) / QT;
    hipLaunchKernelGGL((fa_fwd_varlen<T, OT, D, CAUSAL, PAIR>),
                       dim3((unsigned)(ntiles * a.H * a.S * a.NC)), dim3(kThreads8), 0,
                       a.stream, (const T *)a.q, (const T *)a.k, (const T *)a.v, (OT *)a.o,
                       a.lse, a.cu_q, a.cu_k, a.S, a.H, a.Tq, a.Tk, ntiles, c, neg, a.ws,
                       a.NC, a.KC, a.NT);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.NC == 1) return e;
    constexpr int SPLIT = QT / merge_rows<D>();
    hipLaunchKernelGGL((fa_merge_varlen<OT, D, CAUSAL, QT>),
                       dim3((unsigned)(ntiles * a.H * a.S * SPLIT)), dim3(kThreads), 0,
                       a.stream, (const float *)a.ws, (OT *)a.o, a.lse, a.cu_q, a.cu_k, a.S,
                       a.H, a.Tq, a.Tk, a.NC, a.KC, a.NT);
    return hipGetLastError();
  };
  if constexpr (D == 128)
    return a.pair ? go(std::true_type{}) : go(std::false_type{});
  else
    return go(std::false_type{});
}

template <typename T, typename OT>
hipError_t dispatch_varlen(const VarlenArgs &a, int D, bool causal) {
  switch (D) {
    case 16: return causal ? launch_varlen<T, OT, 16, true>(a) : launch_varlen<T, OT, 16, false>(a);
    case 32: return causal ? launch_varlen<T, OT, 32, true>(a) : launch_varlen<T, OT, 32, false>(a);
    case 64: return causal ? launch_varlen<T, OT, 64, true>(a) : launch_varlen<T, OT, 64, false>(a);
    default:
      return causal ? launch_varlen<T, OT, 128, true>(a) : launch_varlen<T, OT, 128, false>(a);
  }
}

// Shape checks of the varlen entry points (before any pointer is looked at).
int varlen_shape(int64_t S, int64_t H, int64_t Tq, int64_t Tk, int64_t max_seqlen_q,
                 int64_t max_seqlen_k, int64_t D, int dtype) {
  if (S < 1 || H < 1 || Tq < 1 || Tk < 0 || max_seqlen_q < 1 || max_seqlen_k < 0)
    return FA_ERR_SHAPE;
  if (D != 16 && D != 32 && D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  if (dtype != FA_BF16 && dtype != FA_BF16_OF32 && dtype != FA_F16 && dtype != FA_F16_OF32)
    return FA_ERR_DTYPE;
  const int64_t lim = (int64_t)1 << 31;
  // a sequence is addressed like a (batch, head) slice of fa_fwd
  if (Tq > lim / (D * 4) - QRows<false>::value || Tk > lim / (D * 4) - 5 * kBN)
    return FA_ERR_SHAPE;
  const int64_t mq = max_seqlen_q < Tq ? max_seqlen_q : Tq;
  const int64_t ntiles = (mq + kPairRows - 1) / kPairRows;  // the finer tiling
  if (S > lim || H > lim || H * S > lim / ntiles || H * Tq > lim || H * Tk > lim)
    return FA_ERR_SHAPE;
  return FA_OK;
}

// Tile layout and key split of a varlen call.  Layout: at D = 128 the
// pair-split 128-row tiles when the packed rows make fewer 256-row tiles
// than there are compute units (the stream schedule's rule) and sequences
// are long on average (measured on 32768 tokens, causal, unsplit: 8
// sequences +9% with pair-split, 32 sequences -15%: short sequences are
// dominated by the fixed cost of a tile, which the finer tiles double).
// Stream (max_seqlen_k > 0 and H * S <= kVPairs): the units of every
// (head, sequence) pair, counted by each workgroup from the offsets, dealt
// evenly over G workgroups; see the rule in varlen_plan.
// Split (max_seqlen_k > 0, more pairs): the work is at most Tq * max_seqlen_q / 2
// (causal) or Tq * max_seqlen_k row-key pairs, in units of one tile's rows
// by 64 keys; a chunk gets at least that divided by the compute units (and
// at least kMinChunk units, against the fixed cost of a piece), and a tile
// at most kMaxChunks chunks.  Unless the longest tile makes kMinSplit
// chunks, nothing is split.
struct VarlenSplit {
  bool pair;
  int NC, KC, NT;
  int G;            // > 0: stream schedule over G workgroups
  size_t plan_off;  // its cut table in the workspace
  size_t bytes;
};
constexpr int kMinChunk = 8;
constexpr int kMinSplit = 3;
constexpr int kMaxChunks = 16;

int varlen_plan(int64_t S, int64_t H, int64_t Tq, int64_t Tk, int64_t max_seqlen_q,
                int64_t max_seqlen_k, int64_t D, bool causal, VarlenSplit &sp) {
  int cus = 0;
  const int st = device_cus(&cus);
  if (st != FA_OK) return st;
  sp.pair = D == 128 && H * ((Tq + QRows<false>::value - 1) / QRows<false>::value) < cus &&
            Tq / S >= 2048;
  sp.NC = 1;
  sp.KC = 1;
  sp.NT = 1;
  sp.G = 0;
  sp.plan_off = 0;
  sp.bytes = 0;
  if (max_seqlen_k < 1) return FA_OK;
  if (H * S <= kVPairs) {
    // Stream schedule: one workgroup per compute unit (at most kMaxChunks,
    // whose partials the workspace holds).  Pair-split tiles at D = 128 when
    // the packed rows make fewer 256-row tiles than compute units and a
    // compute unit's share of 128 x 64 units, bounded above by taking every
    // sequence as long as the longest, stays under 64 (the dense rule's
    // bound).  Measured on 32768 tokens, causal: 8 sequences of up to 10278
    // tokens (bound 80) ran 8% faster on 256-row tiles, 32 (bound 26) tied,
    // 128 (bound 9) ran 9% faster pair-split.
    const int64_t mq = max_seqlen_q < Tq ? max_seqlen_q : Tq;
    const int64_t mk = max_seqlen_k < Tk ? max_seqlen_k : Tk;
    const int64_t share = H * (causal ? Tq * mq / 2 : Tq * mk) / (kPairRows * kBN);
    sp.pair = D == 128 && H * ((Tq + QRows<false>::value - 1) / QRows<false>::value) < cus &&
              share < 64LL * cus;
    const int64_t QT = sp.pair ? kPairRows : QRows<false>::value;
    sp.G = cus < fa_sched::kMaxChunks ? cus : fa_sched::kMaxChunks;
    sp.plan_off = ((size_t)2 * sp.G * (size_t)QT * (size_t)(D + 4) * 4 + 255) / 256 * 256;
    sp.bytes = sp.plan_off + (size_t)3 * 4 * sp.G;  // the cut table
    return FA_OK;
  }
  const int64_t QT = sp.pair ? kPairRows : QRows<false>::value;
  const int64_t mq = max_seqlen_q < Tq ? max_seqlen_q : Tq;
  const int64_t mk = max_seqlen_k < Tk ? max_seqlen_k : Tk;
  // key tiles of the longest tile
  const int64_t kmax = causal ? (mk < (mq + QT - 1) / QT * QT ? mk : (mq + QT - 1) / QT * QT) : mk;
  const int64_t nkt = (kmax + kBN - 1) / kBN;
  const int64_t pairs = causal ? Tq * mq / 2 : Tq * mk;  // row-key pairs, at most
  const int64_t units = H * (pairs / (QT * kBN) + 1);
  int64_t kc = (units + cus - 1) / cus;
  if (kc < kMinChunk) kc = kMinChunk;
  int64_t nc = (nkt + kc - 1) / kc;
  if (nc > kMaxChunks) nc = kMaxChunks;
  // split only where the longest tile is at least three shares: measured on
  // 32768 tokens, causal, D = 128, two chunks (8 sequences of up to 10278
  // tokens) lost 5% to the extra workgroups and the merge, four (32
  // sequences) gained 9%, seven (one sequence) halved the time
  if (nc < kMinSplit) return FA_OK;
  const int64_t NT = (Tq + QT - 1) / QT + S;
  if (H * NT * nc >= ((int64_t)1 << 31) / QT) return FA_OK;  // slot indices stay in int
  sp.NC = (int)nc;
  sp.KC = (int)kc;
  sp.NT = (int)NT;
  sp.bytes = (size_t)(H * NT * nc) * (size_t)QT * (size_t)(D + 4) * 4;
  return FA_OK;
}

int varlen_entry(const void *q, const void *k, const void *v, void *o, float *lse,
                 const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int64_t S,
                 int64_t H, int64_t Tq, int64_t Tk, int64_t max_seqlen_q, int64_t max_seqlen_k,
                 int64_t D, float scale, int causal, int dtype, void *workspace,
                 size_t workspace_bytes, bool split, void *stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULLPTR;
  int st = varlen_shape(S, H, Tq, Tk, max_seqlen_q, split ? max_seqlen_k : 0, D, dtype);
  if (st != FA_OK) return st;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (max_seqlen_q > Tq) max_seqlen_q = Tq;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGN;
  if (((uintptr_t)lse | (uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k) & 3u)
    return FA_ERR_ALIGN;
  const size_t out_size = (dtype == FA_BF16_OF32 || dtype == FA_F16_OF32) ? 4 : 2;
  const size_t qb = (size_t)(H * Tq * D * 2), kb = (size_t)(H * Tk * D * 2);
  const size_t ob = (size_t)(H * Tq * D) * out_size, lb = (size_t)(H * Tq * 4);
  const size_t cb = (size_t)(S + 1) * 4;
  const void *outs[3] = {o, lse, workspace};
  size_t osz[3] = {ob, lb, 0};
  const void *ins[5] = {q, k, v, cu_seqlens_q, cu_seqlens_k};
  const size_t isz[5] = {qb, kb, kb, cb, cb};
  for (int x = 0; x < 2; ++x)
    for (int y = 0; y < 5; ++y)
      if (overlaps(outs[x], osz[x], ins[y], isz[y])) return FA_ERR_OVERLAP;
  if (overlaps(o, ob, lse, lb)) return FA_ERR_OVERLAP;
  VarlenSplit sp;
  st = varlen_plan(S, H, Tq, Tk, max_seqlen_q, split ? max_seqlen_k : 0, D, causal != 0, sp);
  if (st != FA_OK) return st;
  if (sp.bytes > 0) {
    if (!workspace || workspace_bytes < sp.bytes) return FA_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 15u) return FA_ERR_ALIGN;
    osz[2] = sp.bytes;
    for (int y = 0; y < 5; ++y)
      if (overlaps(workspace, sp.bytes, ins[y], isz[y])) return FA_ERR_OVERLAP;
    for (int x = 0; x < 2; ++x)
      if (overlaps(outs[x], osz[x], workspace, sp.bytes)) return FA_ERR_OVERLAP;
  }
  VarlenArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.S = (int)S;
  a.H = (int)H;
  a.Tq = (int)Tq;
  a.Tk = (int)Tk;
  a.maxq = (int)max_seqlen_q;
  a.pair = sp.pair;
  a.c = scale * 1.4426950408889634f;
  a.ws = sp.bytes > 0 ? (float *)workspace : nullptr;
  a.NC = sp.NC;
  a.KC = sp.KC;
  a.NT = sp.NT;
  a.G = sp.G;
  a.plan_off = sp.plan_off;
  a.stream = (hipStream_t)stream;
  const bool cz = causal != 0;
  hipError_t e;
  switch (dtype) {
    case FA_BF16: e = dispatch_varlen<__bf16, __bf16>(a, (int)D, cz); break;
    case FA_BF16_OF32: e = dispatch_varlen<__bf16, float>(a, (int)D, cz); break;
    case FA_F16: e = dispatch_varlen<_Float16, _Float16>(a, (int)D, cz); break;
    default: e = dispatch_varlen<_Float16, float>(a, (int)D, cz); break;
  }
  if (e != hipSuccess) return hip_fail(e);
  return FA_OK;
}


}  // namespace

// Shared with the backward pass's host code (same library, hidden symbol).
__attribute__((visibility("hidden"))) int fa_internal_hip_fail(hipError_t e) {
  return hip_fail(e);
}

// dQ of fa_bwd on the pipelined kernel (fa_bwd_dq8), for dense problems at
// D = 64 or 128 with 16-bit inputs; called by the backward's host code
// after its row-term kernel.  With fewer than two 128-row query tiles per
// compute unit, and a workspace that holds the plan's partials, it takes the
// stream-K schedule of 128-row tiles (fa_bwd_dq8_stream, then fa_merge_dq8
// for the cut tiles); otherwise one workgroup per tile.
namespace {
constexpr int kDqLead = 3;  // fixed cost of a piece, in 64-key tiles

bool dq8_plan(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, bool causal, int cus,
              StreamPlan &sp) {
  if (D != 64 && D != 128) return false;
  // from two tiles per compute unit on, the grid's longest-first rounds
  // balance as well (measured: B8 N8192 D64 causal 481 us on the grid, 497
  // on the stream schedule; B8 N4096 D128 causal 222 against 198)
  if (BH * ((Nq + 127) / 128) >= 2LL * cus) return false;
  return plan_rows(BH, Nq, Nk, 128, kDqLead, 0, causal, cus, sp);
}

// Split of the masked dQ grid (the rule without causality): a 128-row tile
// that holds global queries sees every key tile, a band tile the global key
// tiles and about (127 + 2 (window - 1)) / 64 band tiles.  Those tiles (the
// first ceil(min(G, Nq) / 128) of each slice) run as S parts of about a
// band tile's list each, at least 32 key tiles; S is limited to what the
// workspace holds, and below 2 they run whole.
struct QSplit {
  int nsp = 0, S = 1;
};
QSplit dq8_split(const Mask &mk, int64_t BH, int64_t Nq, int64_t Nk, int64_t D, size_t avail) {
  QSplit r;
  const int64_t gq = mk.nglobal < Nq ? mk.nglobal : Nq;
  if (mk.causal || gq <= 0 || Nk <= 0) return r;
  const int64_t nkt = (Nk + kBN - 1) / kBN;
  const int64_t gk = mk.nglobal < Nk ? mk.nglobal : Nk;
  int64_t band = (gk + kBN - 1) / kBN + (127 + 2 * ((int64_t)mk.window - 1)) / kBN + 2;
  if (band > nkt) band = nkt;
  const int64_t cap = band > 32 ? band : 32;
  const int64_t nsp = (gq + 127) / 128;
  const size_t per = (size_t)(BH * nsp) * 128 * (size_t)D * 4;  // one part of each
  int64_t S = (nkt + cap - 1) / cap;
  if ((size_t)S > avail / per) S = (int64_t)(avail / per);
  if (S < 2) return r;
  r.nsp = (int)nsp;
  r.S = (int)S;
  return r;
}

template <typename T, typename OT, int D, bool CAUSAL>
hipError_t launch_dq8(const void *q, const void *k, const void *v, const void *o,
                      const void *dout, const float *lse, float *dl, void *dq, int Nq, int Nk,
                      int BH, float c, float scale, const StreamPlan *sp, float *ws,
                      size_t ws_bytes, const Mask *mk, hipStream_t s) {
  if (mk) {  // the window mask: one workgroup per tile (or part) over its key list
    const int nqt = (Nq + 127) / 128;
    const QSplit sl = dq8_split(*mk, BH, Nq, Nk, D, ws ? ws_bytes : 0);
    const int units = nqt + sl.nsp * (sl.S - 1);
    hipLaunchKernelGGL((fa_bwd_dq8<T, OT, D, CAUSAL, true>), dim3((unsigned)(BH * units)),
                       dim3(kThreads8), 0, s, (const T *)q, (const T *)k, (const T *)v,
                       (const T *)o, (const T *)dout, lse, dl, (OT *)dq, ws, Nq, Nk, BH, nqt, c,
                       scale, *mk, sl.nsp, sl.S);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || sl.S < 2) return e;
    hipLaunchKernelGGL((fa_merge_dq8_split<OT, D>),
                       dim3((unsigned)(BH * sl.nsp * (128 / merge_rows<D>()))), dim3(kThreads),
                       0, s, (const float *)ws, (OT *)dq, Nq, scale, BH, sl.nsp, sl.S);
    return hipGetLastError();
  }
  if (sp) {
    ChunkStarts cs;
    CutList cuts;
    make_tables(*sp, CAUSAL, cs, cuts);
    hipLaunchKernelGGL((fa_bwd_dq8_stream<T, OT, D, CAUSAL>), dim3((unsigned)sp->G),
                       dim3(kThreads8), 0, s, (const T *)q, (const T *)k, (const T *)v,
                       (const T *)o, (const T *)dout, lse, dl, (OT *)dq, ws, Nq, Nk, c, scale, *sp, cs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || cuts.n == 0) return e;
    hipLaunchKernelGGL((fa_merge_dq8<OT, D>), dim3((unsigned)(cuts.n * (128 / merge_rows<D>()))),
                       dim3(kThreads), 0, s, (const float *)ws, (OT *)dq, Nq, scale, cuts);
    return hipGetLastError();
  }
  const int nqt = (Nq + 127) / 128;
  hipLaunchKernelGGL((fa_bwd_dq8<T, OT, D, CAUSAL>), dim3((unsigned)(BH * nqt)),
                     dim3(kThreads8), 0, s, (const T *)q, (const T *)k, (const T *)v,
                     (const T *)o, (const T *)dout, lse, dl, (OT *)dq, ws, Nq, Nk, BH, nqt, c,
                     scale, Mask{}, 0, 1);
  return hipGetLastError();
}
template <typename T, typename OT>
hipError_t dq8_d(int D, bool causal, const void *q, const void *k, const void *v,
                 const void *o, const void *dout, const float *lse, float *dl, void *dq, int Nq,
                 int Nk,
                 int BH, float c, float scale, const StreamPlan *sp, float *ws, size_t ws_bytes, const Mask *mk,
                 hipStream_t s) {
  if (D == 64)
    return causal ? launch_dq8<T, OT, 64, true>(q, k, v, o, dout, lse, dl, dq, Nq, Nk, BH, c,
                                                scale, sp, ws, ws_bytes, mk, s)
                  : launch_dq8<T, OT, 64, false>(q, k, v, o, dout, lse, dl, dq, Nq, Nk, BH, c,
                                                 scale, sp, ws, ws_bytes, mk, s);
  return causal ? launch_dq8<T, OT, 128, true>(q, k, v, o, dout, lse, dl, dq, Nq, Nk, BH, c, scale,
                                               sp, ws, ws_bytes, mk, s)
                : launch_dq8<T, OT, 128, false>(q, k, v, o, dout, lse, dl, dq, Nq, Nk, BH, c,
                                                scale, sp, ws, ws_bytes, mk, s);
}
}  // namespace

// dK and dV of fa_bwd on the pipelined kernel (fa_bwd_dkdv8): dense problems
// at D = 64 or 128 with 16-bit inputs, one workgroup per 128-key tile.
namespace {
// Fixed cost of a piece, in 64-row query tiles.  Measured on MI355X
// (causal B8 N4096 D128, B16 N2048 D128, B8 N4096 D64, B2 H8 N2048 D128;
// non-causal B1 H8 N4096 D128) against lead 4: lead 2 gained 1-3% on every
// causal shape and lost 1% on the non-causal one, 6 and 9 the reverse.
constexpr int kKvLead(bool causal) { return causal ? 2 : 6; }

// Stream schedule of fa_bwd_dkdv8_stream: fewer than two 128-key tiles per
// compute unit, and under the causal mask Nq = Nk, a multiple of 128.
bool dkv8_plan(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, bool causal, int cus,
               StreamPlan &sp) {
  if (D != 64 && D != 128) return false;
  if (BH * ((Nk + 127) / 128) >= 2LL * cus) return false;
  if (causal && (Nq != Nk || Nk % 128 != 0)) return false;
  return plan_rows(BH, Nk, Nq, 128, kKvLead(causal), 0, causal, cus, sp);
}

// Split of the masked grid.  A key tile that holds a global key meets every
// query tile from its first key on (every query tile without the causal
// rule), while a band tile meets about (127 + window) / 64 of them (plus the
// global query tiles and the other side of the band without the causal
// rule): one workgroup for such a tile would outlast the whole grid.  Those
// tiles are cut into S parts of about a band tile's list each, at least 32
// query tiles; S is limited to what the workspace holds, and below 2 the
// tiles run whole.
struct KvSplit {
  int nsp = 0;  // split key tiles: [0, nsp) of every slice
  int S = 1;    // parts per split tile
};
KvSplit dkv8_split(const Mask &mk, int64_t BH, int64_t Nq, int64_t Nk, int64_t D,
                   size_t avail) {
  KvSplit r;
  const int64_t g = mk.nglobal < Nk ? mk.nglobal : Nk;
  if (g <= 0 || Nq <= 0) return r;
  const int64_t nqt = (Nq + kBN - 1) / kBN;
  const int64_t w = mk.window;
  const int64_t gq = mk.nglobal < Nq ? mk.nglobal : Nq;
  int64_t band = mk.causal ? (127 + w - 1) / kBN + 2
                           : (gq + kBN - 1) / kBN + (127 + 2 * (w - 1)) / kBN + 2;
  if (band > nqt) band = nqt;
  const int64_t cap = band > 32 ? band : 32;
  const int64_t nsp = (g + 127) / 128;
  const size_t per = (size_t)(BH * nsp) * 2 * 128 * (size_t)D * 4;  // one part of each
  int64_t S = (nqt + cap - 1) / cap;
  if ((size_t)S > avail / per) S = (int64_t)(avail / per);
  if (S < 2) return r;
  r.nsp = (int)nsp;
  r.S = (int)S;
  return r;
}

template <typename T, typename OT, int D, bool CAUSAL>
hipError_t launch_dkv8(const void *q, const void *k, const void *v, const void *dout,
                       const float *lse, const float *dl, void *dk, void *dv, int Nq, int Nk,
                       int BH, float c, float scale, const StreamPlan *sp, float *ws,
                       size_t ws_bytes, const Mask *mk, hipStream_t s) {
  if (mk) {  // the window mask: one workgroup per key tile (or part) over its query list
    const int nkt = (Nk + 127) / 128;
    const KvSplit sl = dkv8_split(*mk, BH, Nq, Nk, D, ws ? ws_bytes : 0);
    const int units = nkt + sl.nsp * (sl.S - 1);
    hipLaunchKernelGGL((fa_bwd_dkdv8<T, OT, D, CAUSAL, true>), dim3((unsigned)(BH * units)),
                       dim3(kThreads8), 0, s, (const T *)q, (const T *)k, (const T *)v,
                       (const T *)dout, lse, dl, (OT *)dk, (OT *)dv, ws, Nq, Nk, BH, nkt, c,
                       scale, *mk, sl.nsp, sl.S);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || sl.S < 2) return e;
    hipLaunchKernelGGL((fa_merge_dkv8_split<OT, D>),
                       dim3((unsigned)(BH * sl.nsp * (128 / merge_rows<D>()))), dim3(kThreads),
                       0, s, (const float *)ws, (OT *)dk, (OT *)dv, Nk, scale, BH, sl.nsp,
                       sl.S);
    return hipGetLastError();
  }
  if (sp) {
    ChunkStarts cs;
    CutList cuts;
    make_tables(*sp, CAUSAL, cs, cuts);
    hipLaunchKernelGGL((fa_bwd_dkdv8_stream<T, OT, D, CAUSAL>), dim3((unsigned)sp->G),
                       dim3(kThreads8), 0, s, (const T *)q, (const T *)k, (const T *)v,
                       (const T *)dout, lse, dl, (OT *)dk, (OT *)dv, ws, Nq, Nk, c, scale, *sp,
                       cs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || cuts.n == 0) return e;
    hipLaunchKernelGGL((fa_merge_dkv8<OT, D>),
                       dim3((unsigned)(cuts.n * (128 / merge_rows<D>()))), dim3(kThreads), 0, s,
                       (const float *)ws, (OT *)dk, (OT *)dv, Nk, scale, sp->nqt, CAUSAL, cuts);
    return hipGetLastError();
  }
  const int nkt = (Nk + 127) / 128;
  hipLaunchKernelGGL((fa_bwd_dkdv8<T, OT, D, CAUSAL>), dim3((unsigned)(BH * nkt)),
                     dim3(kThreads8), 0, s, (const T *)q, (const T *)k, (const T *)v,
                     (const T *)dout, lse, dl, (OT *)dk, (OT *)dv, (float *)nullptr, Nq, Nk, BH,
                     nkt, c, scale, Mask{}, 0, 1);
  return hipGetLastError();
}
template <typename T, typename OT>
hipError_t dkv8_d(int D, bool causal, const void *q, const void *k, const void *v,
                  const void *dout, const float *lse, const float *dl, void *dk, void *dv,
                  int Nq, int Nk, int BH, float c, float scale, const StreamPlan *sp, float *ws,
                  size_t ws_bytes, const Mask *mk, hipStream_t s) {
  if (D == 64)
    return causal ? launch_dkv8<T, OT, 64, true>(q, k, v, dout, lse, dl, dk, dv, Nq, Nk, BH, c,
                                                 scale, sp, ws, ws_bytes, mk, s)
                  : launch_dkv8<T, OT, 64, false>(q, k, v, dout, lse, dl, dk, dv, Nq, Nk, BH,
                                                  c, scale, sp, ws, ws_bytes, mk, s);
  return causal ? launch_dkv8<T, OT, 128, true>(q, k, v, dout, lse, dl, dk, dv, Nq, Nk, BH, c,
                                                scale, sp, ws, ws_bytes, mk, s)
                : launch_dkv8<T, OT, 128, false>(q, k, v, dout, lse, dl, dk, dv, Nq, Nk, BH, c,
                                                 scale, sp, ws, ws_bytes, mk, s);
}
}  // namespace

__attribute__((visibility("hidden"))) bool fa_internal_bwd_dkdv8(
    const void *q, const void *k, const void *v, const void *dout, const float *lse,
    const float *dl, void *dk, void *dv, int Nq, int Nk, int BH, int D, int dtype, bool causal,
    float c, float scale, void *ws, size_t ws_bytes, const int *mask3, void *stream,
    hipError_t *err) {
  if (D != 64 && D != 128) return false;
  Mask mval{};
  const Mask *mk = nullptr;
  if (mask3) {
    // non-causal at D = 128 the window test's three per-lane values push the
    // kernel past 256 VGPRs (a reload inside the loop): the 64-key kernel
    // keeps that case
    if (!mask3[0] && D == 128) return false;
    mval.causal = mask3[0];
    mval.window = mask3[1];
    mval.nglobal = mask3[2];
    mk = &mval;
    causal = mval.causal != 0;  // the kernel's CAUSAL is the rule's
  }
  // One round of 128-key workgroups leaves the causal triangle unbalanced:
  // from two tiles per compute unit on, longest-first rounds balance it
  // (measured: B8 N4096 D128 causal, one tile per unit, 211 us against 201
  // for the 64-key kernel; B1 H16 N8192 968 against 1278); below that the
  // stream schedule, when the workspace holds its partials; else the
  // 64-key kernel.
  int cus = 0;
  if (device_cus(&cus) != FA_OK) return false;
  StreamPlan sp;
  const StreamPlan *use = nullptr;
  if (!mk && (int64_t)BH * ((Nk + 127) / 128) < 2LL * cus) {
    if (!ws || !dkv8_plan(BH, Nq, Nk, D, causal, cus, sp) ||
        ws_bytes < (size_t)2 * sp.G * 2 * 128 * (size_t)D * 4)
      return false;
    use = &sp;
  }
  float *w = (float *)ws;
  hipStream_t s = (hipStream_t)stream;
  switch (dtype) {
    case FA_BF16:
      *err = dkv8_d<__bf16, __bf16>(D, causal, q, k, v, dout, lse, dl, dk, dv, Nq, Nk, BH, c,
                                    scale, use, w, ws_bytes, mk, s);
      return true;
    case FA_BF16_OF32:
      *err = dkv8_d<__bf16, float>(D, causal, q, k, v, dout, lse, dl, dk, dv, Nq, Nk, BH, c,
                                   scale, use, w, ws_bytes, mk, s);
      return true;
    case FA_F16:
      *err = dkv8_d<_Float16, _Float16>(D, causal, q, k, v, dout, lse, dl, dk, dv, Nq, Nk, BH,
                                        c, scale, use, w, ws_bytes, mk, s);
      return true;
    case FA_F16_OF32:
      *err = dkv8_d<_Float16, float>(D, causal, q, k, v, dout, lse, dl, dk, dv, Nq, Nk, BH, c,
                                     scale, use, w, ws_bytes, mk, s);
      return true;
    default: return false;
  }
}

// Bytes of partial sums the splits of the masked dQ and dK/dV grids use for
// this problem and rule (the larger of the two: dQ runs first and dK/dV
// after it; 0 when neither pipelined kernel splits a tile).
__attribute__((visibility("hidden"))) size_t fa_internal_masked_dkv8_bytes(
    int64_t BH, int64_t Nq, int64_t Nk, int64_t D, const int *mask3) {
  if (D != 64 && D != 128) return 0;
  Mask m{};
  m.causal = mask3[0];
  m.window = mask3[1];
  m.nglobal = mask3[2];
  const KvSplit sl = dkv8_split(m, BH, Nq, Nk, D, ~(size_t)0);
  // non-causal at D = 128 dK/dV runs the earlier kernel (no split)
  const bool kv_split = sl.S >= 2 && (mask3[0] || D != 128);
  const size_t kv = kv_split ? (size_t)(BH * sl.nsp) * sl.S * 2 * 128 * (size_t)D * 4 : 0;
  // dQ runs first and dK/dV after it: they share the region
  const QSplit sq = dq8_split(m, BH, Nq, Nk, D, ~(size_t)0);
  const size_t qb = sq.S < 2 ? 0 : (size_t)(BH * sq.nsp) * sq.S * 128 * (size_t)D * 4;
  return kv > qb ? kv : qb;
}

// Bytes of dQ partials the stream schedule may need for this problem on a
// device of up to 256 compute units (0 when it never runs), independent of
// the device, so that the backward's workspace query needs no GPU.
__attribute__((visibility("hidden"))) size_t fa_internal_dq8_bytes(int64_t BH, int64_t Nq,
                                                                   int64_t Nk, int64_t D,
                                                                   bool causal) {
  StreamPlan sp;
  if (!dq8_plan(BH, Nq, Nk, D, causal, fa_sched::kMaxChunks, sp)) return 0;
  return (size_t)2 * sp.G * 128 * (size_t)D * 4;
}

// Bytes of dK/dV partials the stream schedule may need (as
// fa_internal_dq8_bytes: for a device of up to 256 compute units, 0 when
// it never runs).
__attribute__((visibility("hidden"))) size_t fa_internal_dkv8_bytes(int64_t BH, int64_t Nq,
                                                                    int64_t Nk, int64_t D,
                                                                    bool causal) {
  StreamPlan sp;
  if (!dkv8_plan(BH, Nq, Nk, D, causal, fa_sched::kMaxChunks, sp)) return 0;
  return (size_t)2 * sp.G * 2 * 128 * (size_t)D * 4;
}

__attribute__((visibility("hidden"))) bool fa_internal_bwd_dq8(
    const void *q, const void *k, const void *v, const void *o, const void *dout,
    const float *lse, float *dl, void *dq, int Nq, int Nk, int BH, int D, int dtype, bool causal,
    float c, float scale, void *ws, size_t ws_bytes, const int *mask3, void *stream,
    hipError_t *err) {
  if (D != 64 && D != 128) return false;
  Mask mval{};
  const Mask *mk = nullptr;
  if (mask3) {
    mval.causal = mask3[0];
    mval.window = mask3[1];
    mval.nglobal = mask3[2];
    mk = &mval;
    causal = mval.causal != 0;  // the kernel's CAUSAL is the rule's (longest tiles first)
  }
  hipStream_t s = (hipStream_t)stream;
  int cus = 0;
  StreamPlan sp;
  const StreamPlan *use = nullptr;
  if (!mk && ws && device_cus(&cus) == FA_OK && dq8_plan(BH, Nq, Nk, D, causal, cus, sp) &&
      ws_bytes >= (size_t)2 * sp.G * 128 * (size_t)D * 4)
    use = &sp;
  float *w = (float *)ws;
  switch (dtype) {
    case FA_BF16:
      *err = dq8_d<__bf16, __bf16>(D, causal, q, k, v, o, dout, lse, dl, dq, Nq, Nk, BH, c, scale,
                                   use, w, ws_bytes, mk, s);
      return true;
    case FA_BF16_OF32:
      *err = dq8_d<__bf16, float>(D, causal, q, k, v, o, dout, lse, dl, dq, Nq, Nk, BH, c, scale,
                                  use, w, ws_bytes, mk, s);
      return true;
    case FA_F16:
      *err = dq8_d<_Float16, _Float16>(D, causal, q, k, v, o, dout, lse, dl, dq, Nq, Nk, BH, c,
                                       scale, use, w, ws_bytes, mk, s);
      return true;
    case FA_F16_OF32:
      *err = dq8_d<_Float16, float>(D, causal, q, k, v, o, dout, lse, dl, dq, Nq, Nk, BH, c,
                                    scale, use, w, ws_bytes, mk, s);
      return true;
    default: return false;
  }
}

// Scratch of fa_fwd_noalloc: the stream-K schedule's partial results, in a
// file-scope device array (one copy per device, held until the process
// ends) instead of caller memory.  FA_NOALLOC_SCRATCH_BYTES covers every
// plan make_plan and plan32 produce on a device of up to 256 compute units
// (the largest, 2 * 256 chunks * 256 rows * (128 + 4) floats, or 4 * 256
// fp32 slots of 128 rows, is 66 MiB).
static __device__ __align__(256) char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress, with that device current) and kept: in host
// code the array's name is a host-side stand-in, never a device address.
int noalloc_scratch(void **ptr) {
  static void *cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev >= 0 && dev < 64) {
    void *p = __atomic_load_n(&cache[dev], __ATOMIC_ACQUIRE);
    if (p) {
      *ptr = p;
      return FA_OK;
    }
  }
  void *p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return hip_fail(e);
  if (!p) return hip_fail(hipErrorInvalidSymbol);
  // the same address whichever thread looks it up first
  if (dev >= 0 && dev < 64) __atomic_store_n(&cache[dev], p, __ATOMIC_RELEASE);
  *ptr = p;
  return FA_OK;
}

}  // namespace

namespace {

// Validation and plan of the FP8 entry points on the pipelined kernel:
// fa_fwd_fp8's argument rules; the workspace holds V widened to bf16
// (rounded up to 256 bytes), then the stream-K partials when the schedule
// of the 16-bit path with the same shape takes one.
struct Fp8Plan {
  Shape sh;
  StreamPlan pl;
  bool stream = false;
  size_t vbytes = 0, bytes = 0;
  float c = 0.f;
};

int fp8_plan(const void *q, const void *k, const void *v, const void *o, const float *lse,
             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, float scale, float dq,
             float dk, float dv, int causal, int out_f32, bool check_ptrs, Fp8Plan &fp) {
  if (check_ptrs && (!q || !k || !v || !o || !lse)) return FA_ERR_NULLPTR;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  if (!isfinite(scale) || !isfinite(dq) || !isfinite(dk) || !isfinite(dv)) return FA_ERR_SCALE;
  fp.c = scale * dq * dk * 1.4426950408889634f;
  if (!isfinite(fp.c)) return FA_ERR_SCALE;
  if (!sizes_fit(B, H, Nq, Nk, D)) return FA_ERR_SHAPE;
  fp.sh.BH = B * H;
  fp.sh.nqt = (Nq + kBM - 1) / kBM;
  fp.sh.qb = (size_t)(fp.sh.BH * Nq * D);
  fp.sh.kb = (size_t)(fp.sh.BH * Nk * D);
  fp.sh.ob = (size_t)(fp.sh.BH * Nq * D) * (out_f32 ? 4 : 2);
  fp.sh.lb = (size_t)(fp.sh.BH * Nq) * 4;
  if (check_ptrs) {
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGN;
    if ((uintptr_t)lse & 3u) return FA_ERR_ALIGN;
    const Shape &sh = fp.sh;
    if (overlaps(o, sh.ob, q, sh.qb) || overlaps(o, sh.ob, k, sh.kb) ||
        overlaps(o, sh.ob, v, sh.kb) || overlaps(lse, sh.lb, q, sh.qb) ||
        overlaps(lse, sh.lb, k, sh.kb) || overlaps(lse, sh.lb, v, sh.kb) ||
        overlaps(o, sh.ob, lse, sh.lb))
      return FA_ERR_OVERLAP;
  }
  int cus = 0;
  const int st = device_cus(&cus);
  if (st != FA_OK) return st;
  size_t pbytes = 0;
  fp.stream = make_plan(fp.sh.BH, Nq, Nk, D, out_f32 ? FA_BF16_OF32 : FA_BF16, causal != 0,
                        cus, fp.pl, pbytes);
  fp.vbytes = (fp.sh.kb * 2 + 255) / 256 * 256;
  fp.bytes = fp.vbytes + (fp.stream ? pbytes : 0);
  return FA_OK;
}

template <typename OT>
hipError_t dispatch_fp8(const Launch &a, int D, bool causal) {
  if (D == 64)
    return causal ? launch16<__bf16, OT, 64, true, uint8_t>(a)
                  : launch16<__bf16, OT, 64, false, uint8_t>(a);
  return causal ? launch16<__bf16, OT, 128, true, uint8_t>(a)
                : launch16<__bf16, OT, 128, false, uint8_t>(a);
}

}  // namespace

extern "C" {

int fa_version(void) { return 400; }

#if FA_DEBUG_BARRIERS
// include/fa_debug.h: ring-barrier mismatches counted on the current device.
int fa_debug_barrier_faults(unsigned int *count, int reset) {
  if (!count) return FA_ERR_NULLPTR;
  hipError_t e = hipMemcpyFromSymbol(count, HIP_SYMBOL(fa_dbg_faults), sizeof(unsigned int), 0,
                                     hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fa_internal_hip_fail(e);
  if (reset) {
    const unsigned int zero = 0u;
    e = hipMemcpyToSymbol(HIP_SYMBOL(fa_dbg_faults), &zero, sizeof(zero), 0,
                          hipMemcpyHostToDevice);
    if (e != hipSuccess) return fa_internal_hip_fail(e);
  }
  return FA_OK;
}
#endif

const char *fa_status_str(int s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULLPTR: return "null pointer argument";
    case FA_ERR_SHAPE: return "invalid shape (B, H, Nq, Nk must be >= 1 and sizes must fit)";
    case FA_ERR_HEAD_DIM: return "unsupported head dimension (D must be 16, 32, 64 or 128)";
    case FA_ERR_DTYPE: return "unknown dtype";
    case FA_ERR_SCALE: return "scale is not finite";
    case FA_ERR_ALIGN: return "misaligned pointer (q, k, v, o, workspace need 16 bytes, lse 4)";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_OVERLAP: return "output or workspace buffers overlap each other or the inputs";
    case FA_ERR_WORKSPACE: return "workspace missing or smaller than its workspace-size query reports";
    default: return "unknown status";
  }
}

const char *fa_last_hip_error(void) { return g_hip_error; }

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
           int64_t H, int64_t Nq, int64_t Nk, int64_t D, float scale, int causal,
           int dtype, void *stream) {
  Shape sh;
  const int st = validate(q, k, v, o, lse, B, H, Nq, Nk, D, scale, dtype, sh);
  if (st != FA_OK) return st;
  return run(q, k, v, o, lse, Nq, Nk, D, scale, causal, dtype, sh, nullptr, nullptr, stream);
}

// The local-window + global-token forward: validated as fa_fwd (16-bit
// inputs only), the window clamped to max(Nq, Nk) (which already covers
// every |i - j|, and keeps the rule's arithmetic in 32 bits), then one
// workgroup per 256-row query tile of the pipelined kernel over that tile's
// key-tile list (key_list).
static Mask masked_rule(int64_t Nq, int64_t Nk, int causal, int64_t window, int64_t nglobal) {
  const int64_t wmax = Nq > Nk ? Nq : Nk;
  Mask mk;
  mk.causal = causal != 0;
  mk.window = (int)(window < wmax ? window : wmax);
  mk.nglobal = (int)(nglobal < wmax ? nglobal : wmax);  // >= max(Nq, Nk): every token
  return mk;
}

int fa_fwd_masked_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                                 int causal, int64_t window, int64_t nglobal, int dtype,
                                 size_t *bytes) {
  if (!bytes) return FA_ERR_NULLPTR;
  *bytes = 0;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || window < 1 || nglobal < 0) return FA_ERR_SHAPE;
  if (D != 16 && D != 32 && D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  if (dtype <= FA_F32 || dtype > FA_F16_OF32) return FA_ERR_DTYPE;
  if (!sizes_fit(B, H, Nq, Nk, D)) return FA_ERR_SHAPE;
  const Mask mk = masked_rule(Nq, Nk, causal, window, nglobal);
  *bytes = fwd_masked_split_bytes(fwd_masked_split(mk, B * H, Nq, Nk, D, ~(size_t)0), B * H, D);
  return FA_OK;
}

int fa_fwd_masked_ws(const void *q, const void *k, const void *v, void *o, float *lse,
                     int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, float scale,
                     int causal, int64_t window, int64_t nglobal, int dtype, void *workspace,
                     size_t workspace_bytes, void *stream) {
  Shape sh;
  const int st = validate(q, k, v, o, lse, B, H, Nq, Nk, D, scale, dtype, sh);
  if (st != FA_OK) return st;
  if (window < 1 || nglobal < 0) return FA_ERR_SHAPE;
  if (dtype == FA_F32) return FA_ERR_DTYPE;
  if (!workspace) workspace_bytes = 0;
  if (workspace) {
    if ((uintptr_t)workspace & 15u) return FA_ERR_ALIGN;
    if (overlaps(workspace, workspace_bytes, q, sh.qb) ||
        overlaps(workspace, workspace_bytes, k, sh.kb) ||
        overlaps(workspace, workspace_bytes, v, sh.kb) ||
        overlaps(workspace, workspace_bytes, o, sh.ob) ||
        overlaps(workspace, workspace_bytes, lse, sh.lb))
      return FA_ERR_OVERLAP;
  }
  const Mask mk = masked_rule(Nq, Nk, causal, window, nglobal);
  return run(q, k, v, o, lse, Nq, Nk, D, scale, causal, dtype, sh, nullptr, workspace, stream,
             &mk, nullptr, workspace_bytes);
}

int fa_fwd_masked(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                  int64_t H, int64_t Nq, int64_t Nk, int64_t D, float scale, int causal,
                  int64_t window, int64_t nglobal, int dtype, void *stream) {
  return fa_fwd_masked_ws(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, window, nglobal,
                          dtype, nullptr, 0, stream);
}

int fa_fwd_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                          int causal, int dtype, size_t *bytes) {
  if (!bytes) return FA_ERR_NULLPTR;
  *bytes = 0;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  if (D != 16 && D != 32 && D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  if (dtype < FA_F32 || dtype > FA_F16_OF32) return FA_ERR_DTYPE;
  if (!sizes_fit(B, H, Nq, Nk, D)) return FA_ERR_SHAPE;
  int cus = 0;
  const int st = device_cus(&cus);
  if (st != FA_OK) return st;
  StreamPlan pl;
  Split32 ks;
  size_t ws = 0;
  plan_ws(B * H, Nq, Nk, D, dtype, causal != 0, cus, pl, ks, ws);
  *bytes = ws;
  return FA_OK;
}

int fa_fwd_ws(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
              int64_t H, int64_t Nq, int64_t Nk, int64_t D, float scale, int causal,
              int dtype, void *workspace, size_t workspace_bytes, void *stream) {
  Shape sh;
  int st = validate(q, k, v, o, lse, B, H, Nq, Nk, D, scale, dtype, sh);
  if (st != FA_OK) return st;
  if (workspace) {
    if ((uintptr_t)workspace & 15u) return FA_ERR_ALIGN;
    if (overlaps(workspace, workspace_bytes, q, sh.qb) ||
        overlaps(workspace, workspace_bytes, k, sh.kb) ||
        overlaps(workspace, workspace_bytes, v, sh.kb) ||
        overlaps(workspace, workspace_bytes, o, sh.ob) ||
        overlaps(workspace, workspace_bytes, lse, sh.lb))
      return FA_ERR_OVERLAP;
  }
  int cus = 0;
  st = device_cus(&cus);
  if (st != FA_OK) return st;
  StreamPlan pl;
  Split32 ks;
  size_t need = 0;
  if (!plan_ws(sh.BH, Nq, Nk, D, dtype, causal != 0, cus, pl, ks, need))
    return run(q, k, v, o, lse, Nq, Nk, D, scale, causal, dtype, sh, nullptr, nullptr,
               stream);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  return run(q, k, v, o, lse, Nq, Nk, D, scale, causal, dtype, sh,
             dtype == FA_F32 ? nullptr : &pl, workspace, stream, nullptr, &ks);
}

int fa_fwd_fp8_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                              int causal, int out_f32, size_t *bytes) {
  if (!bytes) return FA_ERR_NULLPTR;
  *bytes = 0;
  Fp8Plan fp;
  const int st = fp8_plan(nullptr, nullptr, nullptr, nullptr, nullptr, B, H, Nq, Nk, D, 1.f,
                          1.f, 1.f, 1.f, causal, out_f32, false, fp);
  if (st != FA_OK) return st;
  *bytes = fp.bytes;
  return FA_OK;
}

int fa_fwd_fp8_ws(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                  int64_t H, int64_t Nq, int64_t Nk, int64_t D, float scale, float descale_q,
                  float descale_k, float descale_v, int causal, int out_f32, void *workspace,
                  size_t workspace_bytes, void *stream) {
  Fp8Plan fp;
  int st = fp8_plan(q, k, v, o, lse, B, H, Nq, Nk, D, scale, descale_q, descale_k, descale_v,
                    causal, out_f32, true, fp);
  if (st != FA_OK) return st;
  if (!workspace || workspace_bytes < fp.bytes) return FA_ERR_WORKSPACE;
  if ((uintptr_t)workspace & 15u) return FA_ERR_ALIGN;
  const Shape &sh = fp.sh;
  if (overlaps(workspace, fp.bytes, q, sh.qb) || overlaps(workspace, fp.bytes, k, sh.kb) ||
      overlaps(workspace, fp.bytes, v, sh.kb) || overlaps(workspace, fp.bytes, o, sh.ob) ||
      overlaps(workspace, fp.bytes, lse, sh.lb))
    return FA_ERR_OVERLAP;
  hipStream_t hs = (hipStream_t)stream;
  const size_t n16 = sh.kb / 16;  // D is a multiple of 16
  hipLaunchKernelGGL(fa_fp8_widen, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, hs,
                     (const u32x4 *)v, (u32x4 *)workspace, n16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  Launch a;
  a.masked = false;
  a.mk = Mask{};
  a.q = q;
  a.k = k;
  a.v = workspace;
  a.o = o;
  a.lse = lse;
  a.ws = (float *)((char *)workspace + fp.vbytes);
  a.Nq = (int)Nq;
  a.Nk = (int)Nk;
  a.BH = (int)sh.BH;
  a.nqt = (int)sh.nqt;
  a.nqtg = (int)((Nq + QRows<false>::value - 1) / QRows<false>::value);
  a.c = fp.c;
  a.osc = descale_v;
  a.KC = 0;
  a.nsplit = 1;
  a.stream = hs;
  a.plan = fp.stream ? &fp.pl : nullptr;
  ChunkStarts starts;
  CutList cuts;
  a.starts = nullptr;
  a.cuts = nullptr;
  if (fp.stream) {
    make_tables(fp.pl, causal != 0, starts, cuts);
    a.starts = &starts;
    a.cuts = &cuts;
  }
  e = out_f32 ? dispatch_fp8<float>(a, (int)D, causal != 0)
              : dispatch_fp8<__bf16>(a, (int)D, causal != 0);
  if (e != hipSuccess) return hip_fail(e);
  return FA_OK;
}

int fa_fwd_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                   int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, float scale,
                   int causal, int dtype, void *stream) {
  Shape sh;
  int st = validate(q, k, v, o, lse, B, H, Nq, Nk, D, scale, dtype, sh);
  if (st != FA_OK) return st;
  int cus = 0;
  st = device_cus(&cus);
  if (st != FA_OK) return st;
  StreamPlan pl;
  Split32 ks;
  size_t need = 0;
  if (!plan_ws(sh.BH, Nq, Nk, D, dtype, causal != 0, cus, pl, ks, need))
    return run(q, k, v, o, lse, Nq, Nk, D, scale, causal, dtype, sh, nullptr, nullptr,
               stream);
  if (need > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
  void *ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != FA_OK) return st;
  return run(q, k, v, o, lse, Nq, Nk, D, scale, causal, dtype, sh,
             dtype == FA_F32 ? nullptr : &pl, ws, stream, nullptr, &ks);
}

int fa_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                  const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int64_t S,
                  int64_t H, int64_t Tq, int64_t Tk, int64_t max_seqlen_q, int64_t D,
                  float scale, int causal, int dtype, void *stream) {
  return varlen_entry(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, S, H, Tq, Tk, max_seqlen_q,
                      0, D, scale, causal, dtype, nullptr, 0, false, stream);
}

int fa_fwd_varlen_workspace_size(int64_t S, int64_t H, int64_t Tq, int64_t Tk,
                                 int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t D,
                                 int causal, int dtype, size_t *bytes) {
  if (!bytes) return FA_ERR_NULLPTR;
  *bytes = 0;
  int st = varlen_shape(S, H, Tq, Tk, max_seqlen_q, max_seqlen_k, D, dtype);
  if (st != FA_OK) return st;
  VarlenSplit sp;
  st = varlen_plan(S, H, Tq, Tk, max_seqlen_q, max_seqlen_k, D, causal != 0, sp);
  if (st != FA_OK) return st;
  *bytes = sp.bytes;
  return FA_OK;
}

int fa_fwd_varlen_ws(const void *q, const void *k, const void *v, void *o, float *lse,
                     const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int64_t S,
                     int64_t H, int64_t Tq, int64_t Tk, int64_t max_seqlen_q,
                     int64_t max_seqlen_k, int64_t D, float scale, int causal, int dtype,
                     void *workspace, size_t workspace_bytes, void *stream) {
  return varlen_entry(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, S, H, Tq, Tk, max_seqlen_q,
                      max_seqlen_k, D, scale, causal, dtype, workspace, workspace_bytes, true,
                      stream);
}

}  // extern "C"
