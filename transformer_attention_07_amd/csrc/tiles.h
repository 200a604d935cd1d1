// tiles.h -- MFMA tile helpers of the backward kernels (fa_bwd.hip) and the
// FP8 forward (fa_fp8.hip): v_mfma_f32_32x32x16 on
// 16-bit operands, LDS images of 128-row blocks, register-staged loads,
// row-wise and transposed (ds_read_b64_tr_b16) A-operand fragments, and
// stores of transposed 32x32 accumulators.  Each including file keeps its
// own copy in an anonymous namespace.
#ifndef FA_TILES_H
#define FA_TILES_H

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "mask.h"
#include "mma16.h"

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kOwn = 32;  // keys / queries owned by one wave
// Workgroups of four waves: two groups of 32 keys (or queries), and two
// parities that split each streamed block between them, summed at the end.
// 64 keys per workgroup make causal problems twice as many, finer
// workgroups, issued longest first, so the compute units stay evenly loaded
// (a wave has a SIMD to itself: its accumulators need more than 256
// registers at D = 128).
constexpr int kTile = 2 * kOwn;  // keys / queries per workgroup
// Rows per block streamed through LDS: four 32-row quarters, two per wave,
// so one quarter's MFMAs can run beside the other's exponentials.
constexpr int kBlk = 128;
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) float lds_float;

// LDS image of one block of kBlk rows of a [N, D] 16-bit tensor, row-major.
// The row stride (in bytes) is 16 * odd, so the 16 rows of one ds_read_b128
// pass start on distinct 16-byte bank groups, and the four rows of one
// ds_read_b64_tr_b16 group land on disjoint 32-byte ranges.
template <int D> struct Blk {
  static constexpr int STRIDE = D == 128 ? 304 : D == 64 ? 208 : 112;  // D <= 32: 112
  static constexpr int BYTES = kBlk * STRIDE;
};

// Register staging of one block: global -> VGPRs -> LDS, 16 bytes a piece.
template <int D, int ROWS = kBlk> struct Stage {
  static constexpr int CPR = D / 8;  // 16-byte pieces per row
  static constexpr int PIECES = ROWS * CPR;
  static constexpr int N = (PIECES + kThreads - 1) / kThreads;
  u32x4 r[N];

  // rows row0 .. row0+ROWS-1 of a slice with nrows rows; missing rows are 0
  __device__ __forceinline__ void load(const void *slice, int row0, int nrows, int tid) {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int c = tid + n * kThreads;
      r[n] = u32x4{0u, 0u, 0u, 0u};
      if (c < PIECES) {
        const int row = row0 + c / CPR;
        if (row < nrows)
          r[n] = *(const u32x4 *)((const char *)slice + (size_t)row * (D * 2) + (c % CPR) * 16);
      }
    }
  }
  __device__ __forceinline__ void store(lds_char *dst, int tid) const {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int c = tid + n * kThreads;
      if (c < PIECES)
        *(lds_u32x4 *)(dst + (c / CPR) * Blk<D>::STRIDE + (c % CPR) * 16) = r[n];
    }
  }
};

__device__ __forceinline__ u32x2 read_tr16(const lds_char *p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
  return __builtin_bit_cast(u32x2, r);
}

// A operand (32 x 16, rows = head-dim columns d0 .. d0+31 of the block,
// contraction = 16 block rows r0 ..) read transposed from a row-major LDS
// block.  Contraction slot e of half-wave g holds block row
// r0 + 8*(e/4) + 4*g + e%4, the row order of a 32x32 accumulator's
// registers 8*t' .. 8*t'+7, so the matching B operand is those registers.
template <typename T, int D>
__device__ __forceinline__ typename Mma<T>::frag tr_frag(const lds_char *blk, int r0, int d0,
                                                       int lane) {
  const int s = lane & 15, g16 = (lane >> 4) & 1, g = lane >> 5;
  const lds_char *p =
      blk + (r0 + 4 * g + (s >> 2)) * Blk<D>::STRIDE + (d0 + 16 * g16 + 4 * (s & 3)) * 2;
  const u32x2 lo = read_tr16(p);
  const u32x2 hi = read_tr16(p + 8 * Blk<D>::STRIDE);
  const u32x4 raw = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(typename Mma<T>::frag, raw);
}

// A operand read row-wise: lane l holds block row r0 + l%32, columns
// d0 + 8*(l/32) .. +7.
template <typename T, int D>
__device__ __forceinline__ typename Mma<T>::frag row_frag(const lds_char *blk, int r0, int d0,
                                                        int lane) {
  const lds_char *p =
      blk + (r0 + (lane & 31)) * Blk<D>::STRIDE + (d0 + 8 * (lane >> 5)) * 2;
  return __builtin_bit_cast(typename Mma<T>::frag, *(const lds_u32x4 *)p);
}

// Registers 8t' .. 8t'+7 of an accumulator, rounded to T, as a B operand.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag pack_b(const float *x) {
  const u32x4 raw = {Mma<T>::pack2(x[0], x[1]), Mma<T>::pack2(x[2], x[3]),
                     Mma<T>::pack2(x[4], x[5]), Mma<T>::pack2(x[6], x[7])};
  return __builtin_bit_cast(typename Mma<T>::frag, raw);
}

// Row `row` (or zeros past nrows) of a [N, D] slice: 16 bytes at column d0.
template <typename T, int D>
__device__ __forceinline__ typename Mma<T>::frag glob_frag(const T *slice, int row, int nrows,
                                                         int d0) {
  u32x4 raw = {0u, 0u, 0u, 0u};
  if (row < nrows) raw = *(const u32x4 *)(slice + (size_t)row * D + d0);
  return __builtin_bit_cast(typename Mma<T>::frag, raw);
}

template <typename OT> __device__ __forceinline__ void store4(OT *dst, f32x4 x);
template <> __device__ __forceinline__ void store4<float>(float *dst, f32x4 x) {
  *(f32x4 *)dst = x;
}
template <> __device__ __forceinline__ void store4<__bf16>(__bf16 *dst, f32x4 x) {
  const u32x2 w = {Mma<__bf16>::pack2(x[0], x[1]), Mma<__bf16>::pack2(x[2], x[3])};
  *(u32x2 *)dst = w;
}
template <> __device__ __forceinline__ void store4<_Float16>(_Float16 *dst, f32x4 x) {
  const u32x2 w = {Mma<_Float16>::pack2(x[0], x[1]), Mma<_Float16>::pack2(x[2], x[3])};
  *(u32x2 *)dst = w;
}

// Stores a 32 x 32 accumulator holding rows d = d0 + 8(r/4) + 4g + r%4 of a
// transposed gradient for the lane's row `row` of the [N, D] output, times
// `mul`.
template <typename OT, int D>
__device__ __forceinline__ void store_t(OT *slice, int row, int d0, int g, const f32x16 &acc,
                                        float mul) {
  // D = 16: rows 16..31 of the single chunk came from zero padding; skipped
#pragma unroll
  for (int r4 = 0; r4 < (D < 32 ? 2 : 4); ++r4) {
    const f32x4 x = {acc[4 * r4] * mul, acc[4 * r4 + 1] * mul, acc[4 * r4 + 2] * mul,
                     acc[4 * r4 + 3] * mul};
    store4<OT>(slice + (size_t)row * D + d0 + 8 * r4 + 4 * g, x);
  }
}

// 32-row output chunks along the head dimension (one, half padding, at D = 16)
template <int D> constexpr int chunks() { return D < 32 ? 1 : D / 32; }

// At D = 16 the LDS rows are 32 columns wide (the transposed reads of the
// 32-row output MFMAs cover 32 columns) and columns 16..31 must read as zero;
// the blocks never write them, so they are cleared once, before any block
// is stored (the caller then synchronises).
template <int D>
__device__ __forceinline__ void clear_padding(lds_char *smem, int bytes, int tid) {
  if constexpr (D < 32) {
    for (int o = tid * 16; o < bytes; o += kThreads * 16)
      *(lds_u32x4 *)(smem + o) = u32x4{0u, 0u, 0u, 0u};
  }
}

}  // namespace

#endif  // FA_TILES_H
