// mask.h -- the local-window + global-token visibility rule of
// fa_fwd_masked and fa_bwd_masked, as host + device code so that the kernels
// and a host check (plain C++ when not compiled as HIP) run the same tests.
//
// The rule is the reading used here of the sparse attention that combines
// local windows with global tokens, which page "FlashAttention-2实现与优化：
// 高效注意力机制详解" §7 names as an extension and page "解释FlashAttention的
// 显存优化原理" §二 uses on long sequences; neither defines the pattern.
// Key j is visible to query i iff
//     (causal ? 0 <= i - j < window : |i - j| < window)        local band
//  or (j < nglobal || i < nglobal) && (!causal || j <= i)       global tokens.
// `any` and `all` answer the question for a whole block of queries x keys;
// the kernels skip blocks for which `any` is false and drop the per-score
// mask where `all` is true.  `any` must never be false for a block with a
// visible pair and `all` never true for a block with a hidden one.
#ifndef FA_MASK_H
#define FA_MASK_H

#if defined(__HIP__)
#define FA_MASK_FN __host__ __device__ __forceinline__
#else
#define FA_MASK_FN inline
#endif

namespace {

struct Mask {
  int causal, window, nglobal;  // window >= 1, nglobal >= 0

  FA_MASK_FN bool visible(int i, int j) const {
    const int d = i - j;
    const bool local = causal ? (d >= 0 && d < window) : (d > -window && d < window);
    const bool global = (j < nglobal || i < nglobal) && (!causal || j <= i);
    return local || global;
  }
  // The band alone: visible(i, j) for i, j >= nglobal, where the global part
  // is false.  One subtraction and one unsigned compare: i - j wraps to a
  // large value when negative (causal), and |d| < window is d + window - 1
  // in [0, 2 window - 2].  Exact while |i - j| + 3 window < 2^32 (callers
  // clamp window to max(Nq, Nk)).
  FA_MASK_FN bool band(int i, int j) const {
    const unsigned d = (unsigned)(i - j);
    return causal ? d < (unsigned)window
                  : d + (unsigned)(window - 1) < 2u * (unsigned)window - 1u;
  }
  // Is some pair of queries [ilo, ihi] x keys [jlo, jhi] visible?  Exact:
  // i - j takes every value in [ilo - jhi, ihi - jlo], so the band is hit iff
  // that interval meets it.  Global part: the lowest key jlo against the
  // highest query ihi; under causality a global query i sees only keys
  // j <= i < nglobal, which are global keys already.
  FA_MASK_FN bool any(int ilo, int ihi, int jlo, int jhi) const {
    const bool gk = jlo < nglobal && (!causal || jlo <= ihi);
    const bool gq = !causal && ilo < nglobal;
    const bool local = causal ? (ihi - jlo >= 0 && ilo - jhi <= window - 1)
                              : (ihi - jlo >= -(window - 1) && ilo - jhi <= window - 1);
    return gk || gq || local;
  }
  // Is every pair of queries [ilo, ihi] x keys [jlo, jhi] visible?  A
  // sufficient test: one part of the rule covers the whole block.
  FA_MASK_FN bool all(int ilo, int ihi, int jlo, int jhi) const {
    const bool cz = !causal || jhi <= ilo;
    const bool local = causal ? (ilo - jhi >= 0 && ihi - jlo <= window - 1)
                              : (ihi - jlo <= window - 1 && jhi - ilo <= window - 1);
    return local || ((jhi < nglobal || ihi < nglobal) && cz);
  }
};

}  // namespace

#endif  // FA_MASK_H
