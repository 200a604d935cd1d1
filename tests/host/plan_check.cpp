// Host check of the stream-K schedule of fa_fwd_ws (make_plan, ChunkWalk,
// CutTile, make_tables of csrc/stream_plan.h, the code the kernels and the
// host planner run), and of the backward's plans of 128-row and 128-key
// tiles (plan_rows): for many shapes, lead and tail units and
// compute-unit counts, every key tile of every query tile is covered by
// exactly one piece, pieces that do not cover their whole tile write to
// distinct workspace slots, those tiles are exactly the cut list, the
// merge's enumeration of each cut tile yields exactly its pieces, whose key
// ranges partition the tile, and the host tables the kernels read (chunk
// starts, cut tiles with their slots) agree with ChunkWalk::init and
// CutTile.  Prints "ok <plans checked>" or the first
// failure; exit status 0 on success.
#include "../../transformer_attention_07_amd/csrc/stream_plan.h"

#include <cstdio>
#include <map>
#include <set>
#include <tuple>
#include <vector>

using namespace fa_sched;

namespace {

struct Piece {
  int ch, kt0, kt1, slot;
};

// rows128: the plan of the backward's 128-row (dQ) or 128-key (dK/dV)
// tiles, plan_rows with lead `lead` instead of make_plan's.
int check(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, bool causal, int cus, int lead,
          int tail, bool rows128 = false) {
  StreamPlan sp;
  size_t ws = 0;
  if (rows128) {
    if (!plan_rows(BH, Nq, Nk, 128, lead, 0, causal, cus, sp)) return 0;
    lead = -1;
    ws = (size_t)2 * sp.G * 128 * (size_t)(D + 4) * 4;
  } else if (!make_plan(BH, Nq, Nk, D, FA_BF16, causal, cus, sp, ws)) {
    return 0;
  }
  if (lead >= 0) {  // the same plan with other lead and tail units
    sp.lead = lead;
    sp.tail = tail;
    sp.per_head =
        prefix_nat(sp.nqt, sp.nkt, sp.tu, causal) + (long long)(sp.lead + sp.tail) * sp.nqt;
    sp.T = BH * sp.per_head;
    const int gmax = cus < kMaxChunks ? cus : kMaxChunks;
    sp.G = (int)(sp.T < gmax ? sp.T : gmax);
    sp.cq = sp.T / sp.G;
    sp.cr = (int)(sp.T % sp.G);
  }
  const int qt = sp.tu * kKeys;
  auto fail = [&](const char *what, long long a, long long b) {
    printf("FAIL %s (%lld, %lld): BH=%lld Nq=%lld Nk=%lld D=%lld causal=%d cus=%d lead=%d "
           "tail=%d G=%d\n",
           what, a, b, (long long)BH, (long long)Nq, (long long)Nk, (long long)D, (int)causal,
           cus, sp.lead, sp.tail, sp.G);
    return -1;
  };
  if (sp.nqt != (int)((Nq + qt - 1) / qt)) return fail("nqt", sp.nqt, qt);
  if (ws != (size_t)2 * sp.G * qt * (size_t)(D + 4) * 4 && lead < 0) return fail("ws", (long long)ws, 0);
  ChunkStarts cs;
  CutList tab;
  make_tables(sp, causal, cs, tab);
  std::map<std::pair<int, int>, std::vector<Piece>> tiles;  // (bh, t) -> pieces
  std::set<int> slots;
  for (int ch = 0; ch < sp.G; ++ch) {
    ChunkWalk cw;
    cw.init(sp, ch, causal);
    ChunkWalk tw;  // the kernels' start, from the host table
    tw.init_at(sp, ch, cs.w[2 * ch], cs.w[2 * ch + 1]);
    if (tw.bh != cw.bh || tw.zo != cw.zo || tw.u != cw.u || tw.left != cw.left)
      return fail("chunk start table", ch, tw.u);
    PipeItem it;
    int t;
    while (cw.next(sp, causal, it, t)) {
      if (it.bh < 0 || it.bh >= BH || t < 0 || t >= sp.nqt) return fail("tile", it.bh, t);
      if (it.slot >= 0) {
        if (it.slot != 2 * ch && it.slot != 2 * ch + 1) return fail("slot owner", it.slot, ch);
        if (!slots.insert(it.slot).second) return fail("slot reused", it.slot, ch);
      }
      tiles[{it.bh, t}].push_back({ch, it.kt0, it.kt1, it.slot});
    }
  }
  std::set<std::pair<int, int>> partial;
  for (int bh = 0; bh < BH; ++bh)
    for (int t = 0; t < sp.nqt; ++t) {
      const int w = tile_w(t, sp.nkt, sp.tu, causal);
      auto itr = tiles.find({bh, t});
      if (itr == tiles.end()) return fail("tile missing", bh, t);
      std::vector<int> cover(w, 0);
      for (const Piece &p : itr->second) {
        if (p.kt0 < 0 || p.kt1 > w || p.kt0 >= p.kt1) return fail("range", p.kt0, p.kt1);
        for (int x = p.kt0; x < p.kt1; ++x) cover[x]++;
        if ((p.slot < 0) != (p.kt0 == 0 && p.kt1 == w)) return fail("full/slot", p.kt0, p.slot);
      }
      for (int x = 0; x < w; ++x)
        if (cover[x] != 1) return fail("coverage", t, x);
      if (itr->second.size() > 1) partial.insert({bh, t});
      else if (itr->second[0].slot >= 0) return fail("lone partial", bh, t);
    }
  // The cut tiles by CutTile (every boundary j) against the host table,
  // which lists the same tiles in boundary order with the same slots; both
  // must give exactly the pieces of the walk.
  std::vector<int> cut_js;
  for (int j = 1; j < sp.G; ++j) {
    CutTile ct;
    ct.init(sp, j, causal);
    if (ct.cut) cut_js.push_back(j);
  }
  if ((int)cut_js.size() != tab.n) return fail("cut count", (long long)cut_js.size(), tab.n);
  std::set<std::pair<int, int>> listed;
  for (int i = 0; i < tab.n; ++i) {
    CutTile ct;
    ct.init(sp, cut_js[i], causal);
    const uint32_t w0 = tab.w[2 * i], w1 = tab.w[2 * i + 1];
    if ((int)(w0 & 0xffffu) != ct.bh || (int)(w0 >> 16) != ct.t || (int)(w1 & 0xffffu) != ct.j)
      return fail("cut table entry", i, ct.j);
    if (!listed.insert({ct.bh, ct.t}).second) return fail("cut listed twice", ct.bh, ct.t);
    std::set<int> want;
    for (const Piece &p : tiles[{ct.bh, ct.t}]) want.insert(p.slot);
    std::set<int> got, got_tab;
    for (int cc = ct.j - 1;; ++cc) {
      const int s = ct.slot(sp, cc);
      if (s < 0) break;
      got.insert(s);
    }
    for (int k = 0; k < cut_pieces(w1); ++k) got_tab.insert(cut_slot(w1, k));
    if (got != want) return fail("merge pieces", ct.bh, ct.t);
    if (got_tab != want || (int)got_tab.size() != cut_pieces(w1))
      return fail("merge pieces (table)", ct.bh, ct.t);
  }
  if (listed != partial) return fail("cut set", (long long)listed.size(), (long long)partial.size());
  return 1;
}

// Key chunks of a split variable-length tile (varlen_split): for every tile
// length, chunk cap and minimum chunk length the kernels can meet, the
// chunks [i*kc, min((i+1)*kc, nkt)) for i < count are non-empty and cover
// the tile's key tiles exactly once, there are at most NC of them, and
// wherever the earlier rule (count = min(NC, ceil(nkt / KC))) left no chunk
// empty the count is unchanged.
int check_varlen_split() {
  int n = 0;
  for (int NC = 1; NC <= 16; ++NC)
    for (int KC = 1; KC <= 64; ++KC)
      for (int nkt = 1; nkt <= 1024; ++nkt) {
        int kc = 0;
        const int nch = varlen_split(nkt, NC, KC, kc);
        if (nch < 1 || nch > NC || kc < 1) {
          printf("FAIL varlen_split count: nkt=%d NC=%d KC=%d -> %d chunks of %d\n", nkt, NC,
                 KC, nch, kc);
          return -1;
        }
        int covered = 0;
        for (int i = 0; i < nch; ++i) {
          const int a = i * kc, b = (a + kc < nkt) ? a + kc : nkt;
          if (a != covered || b <= a) {
            printf("FAIL varlen_split chunk %d: nkt=%d NC=%d KC=%d kc=%d\n", i, nkt, NC, KC,
                   kc);
            return -1;
          }
          covered = b;
        }
        if (covered != nkt) {
          printf("FAIL varlen_split cover: nkt=%d NC=%d KC=%d\n", nkt, NC, KC);
          return -1;
        }
        int old = (nkt + KC - 1) / KC;
        if (old > NC) old = NC;
        const int kold = (nkt + old - 1) / old;
        if ((old - 1) * kold < nkt && old != nch) {
          printf("FAIL varlen_split changed: nkt=%d NC=%d KC=%d\n", nkt, NC, KC);
          return -1;
        }
        ++n;
      }
  return n;
}

}  // namespace

int main() {
  int n = check_varlen_split();
  if (n < 0) return 1;
  const int64_t Ns[] = {1, 33, 64, 127, 128, 129, 255, 256, 300, 1000, 2048, 3000, 4096, 8192};
  const int cuss[] = {1, 3, 8, 80, 256, 304, 1024};
  const int leads[][2] = {{-1, 0}, {0, 0}, {1, 0}, {5, 0}, {17, 0}, {0, 3}, {5, 2}, {6, 9}};
  for (int64_t BH : {1, 2, 3, 8})
    for (int64_t Nq : Ns)
      for (int64_t Nk : {(int64_t)1, (int64_t)63, (int64_t)500, (int64_t)4096, Nq})
        for (int64_t D : {16, 32, 64, 128})
          for (int causal = 0; causal < 2; ++causal)
            for (int cus : cuss)
              for (const auto &lt : leads) {
                const int r = check(BH, Nq, Nk, D, causal != 0, cus, lt[0], lt[1]);
                if (r < 0) return 1;
                n += r;
              }
  for (int64_t BH : {1, 2, 3, 8, 40})
    for (int64_t Nq : Ns)
      for (int64_t Nk : {(int64_t)1, (int64_t)500, Nq})
        for (int causal = 0; causal < 2; ++causal)
          for (int cus : cuss)
            for (int lead : {0, 3, 4}) {
              const int r = check(BH, Nq, Nk, 128, causal != 0, cus, lead, 0, true);
              if (r < 0) return 1;
              n += r;
            }
  printf("ok %d\n", n);
  return 0;
}
