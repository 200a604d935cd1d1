// Host check of the block tests of the local-window + global-token mask
// (Mask::any and Mask::all of csrc/mask.h, the code the masked kernels run):
// for every small window, global count and causal flag and every block of
// queries x keys in a small square, `any` equals the brute-force "some pair is
// visible" (it is meant to be exact) and `all` never holds for a block with a
// hidden pair; it also holds for every single visible pair and for every
// block the local band or the global part covers on its own.  The block
// sizes the kernels use (32, 64, 128) are checked on larger offsets, and the
// band-only test (Mask::band) equals the rule wherever the global part is
// out of play.  Prints
// "ok <blocks checked>" or the first failure; exit status 0 on success.
#include "../../transformer_attention_07_amd/csrc/mask.h"

#include <cstdio>
#include <initializer_list>

namespace {

long long checked = 0;

bool brute_any(const Mask &m, int ilo, int ihi, int jlo, int jhi) {
  for (int i = ilo; i <= ihi; ++i)
    for (int j = jlo; j <= jhi; ++j)
      if (m.visible(i, j)) return true;
  return false;
}

bool brute_all(const Mask &m, int ilo, int ihi, int jlo, int jhi) {
  for (int i = ilo; i <= ihi; ++i)
    for (int j = jlo; j <= jhi; ++j)
      if (!m.visible(i, j)) return false;
  return true;
}

// Is the block covered by the band alone or by the global part alone?
bool one_part_covers(const Mask &m, int ilo, int ihi, int jlo, int jhi) {
  bool band = true, glob = true;
  for (int i = ilo; i <= ihi; ++i)
    for (int j = jlo; j <= jhi; ++j) {
      const int d = i - j;
      band = band && (m.causal ? (d >= 0 && d < m.window) : (d > -m.window && d < m.window));
      glob = glob && (j < m.nglobal || i < m.nglobal) && (!m.causal || j <= i);
    }
  return band || glob;
}

int check_block(const Mask &m, int ilo, int ihi, int jlo, int jhi) {
  ++checked;
  const bool a = m.any(ilo, ihi, jlo, jhi), ba = brute_any(m, ilo, ihi, jlo, jhi);
  const bool l = m.all(ilo, ihi, jlo, jhi), bl = brute_all(m, ilo, ihi, jlo, jhi);
  const bool cover = one_part_covers(m, ilo, ihi, jlo, jhi);
  if (a != ba || (l && !bl) || (cover && !l) || (ilo == ihi && jlo == jhi && bl != l)) {
    std::printf("FAIL causal=%d window=%d nglobal=%d queries [%d,%d] keys [%d,%d]: "
                "any=%d brute_any=%d all=%d brute_all=%d one_part=%d\n",
                m.causal, m.window, m.nglobal, ilo, ihi, jlo, jhi, a, ba, l, bl, cover);
    return 1;
  }
  return 0;
}

// The band test against the full rule where the global part is out of play
// (i, j >= nglobal), over small windows and large offsets both ways.
int check_band() {
  const int windows[] = {1, 2, 3, 31, 32, 33, 512, 4096, 1 << 20, 1 << 22};
  const int offs[] = {0, 1, 5, 100, 4095, 65536, (1 << 22) - 1};
  for (int causal = 0; causal < 2; ++causal)
    for (int w : windows)
      for (int ng : {0, 7}) {
        const Mask m{causal, w, ng};
        for (int base : offs)
          for (int a = 0; a < 40; ++a)
            for (int b = 0; b < 40; ++b) {
              const int i = ng + base + a, j = ng + b;
              const int i2 = ng + a, j2 = ng + base + b;  // keys far ahead
              for (int t = 0; t < 2; ++t) {
                const int x = t ? i2 : i, y = t ? j2 : j;
                ++checked;
                if (m.band(x, y) != m.visible(x, y)) {
                  std::printf("FAIL band causal=%d window=%d nglobal=%d i=%d j=%d\n", causal,
                              w, ng, x, y);
                  return 1;
                }
              }
            }
      }
  return 0;
}

}  // namespace

int main() {
  if (check_band()) return 1;
  // Every block inside a 14 x 14 square, all small masks.
  const int n = 14;
  for (int causal = 0; causal < 2; ++causal)
    for (int window = 1; window <= 16; ++window)
      for (int ng = 0; ng <= 15; ++ng) {
        const Mask m{causal, window, ng};
        for (int ilo = 0; ilo < n; ++ilo)
          for (int ihi = ilo; ihi < n; ++ihi)
            for (int jlo = 0; jlo < n; ++jlo)
              for (int jhi = jlo; jhi < n; ++jhi)
                if (check_block(m, ilo, ihi, jlo, jhi)) return 1;
      }
  // Aligned blocks of the kernels' sizes at larger offsets.
  const int sizes[] = {32, 64, 128};
  const int windows[] = {1, 31, 32, 33, 64, 100, 128, 257, 1000};
  const int globals[] = {0, 1, 31, 32, 64, 100, 129};
  for (int causal = 0; causal < 2; ++causal)
    for (int w : windows)
      for (int ng : globals) {
        const Mask m{causal, w, ng};
        for (int bq : sizes)
          for (int bk : sizes)
            for (int i0 = 0; i0 < 1200; i0 += bq)
              for (int j0 = 0; j0 < 1200; j0 += bk)
                if (check_block(m, i0, i0 + bq - 1, j0, j0 + bk - 1)) return 1;
      }
  // Blocks cut short by a ragged tail.
  for (int causal = 0; causal < 2; ++causal)
    for (int w : windows)
      for (int ng : globals) {
        const Mask m{causal, w, ng};
        for (int i0 = 0; i0 < 600; i0 += 32)
          for (int j0 = 0; j0 < 600; j0 += 64)
            for (int cut = 1; cut < 64; cut += 13)
              if (check_block(m, i0, i0 + 31, j0, j0 + cut - 1)) return 1;
      }
  std::printf("ok %lld\n", checked);
  return 0;
}
