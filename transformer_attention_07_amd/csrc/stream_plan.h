// Stream-K schedule of fa_fwd_ws: host and device code shared by the
// kernels of fa_fwd.hip, the host planner and the host check of the
// schedule (plain C++ when not compiled as HIP).
//
// Splitting the key range of one query tile over workgroups and combining
// the parts with the online-softmax rescaling is the sequence parallelism of
// page "FlashAttention技术演进全景图" §3.2, with the update rule of page
// "FlashAttention-2实现与优化：高效注意力机制详解" §3.1.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "fa.h"

#if defined(__HIP__)
#define FA_HD __host__ __device__
#else
#define FA_HD
#endif

namespace fa_sched {

constexpr int kKeys = 64;        // keys per key tile (a unit)
constexpr int kPairRows = 128;   // query rows of a tile, pair-split layout
constexpr int kGridRows = 256;   // query rows of a tile, 256-row layout

// The work of one workgroup: query rows [q0, q0 + rows) of head bh against
// key tiles [kt0, kt1) (64 keys each).  slot < 0: the item covers every key
// the rows see and writes O and L; slot >= 0: the item is one part of a
// split key range and writes a partial result to workspace slot `slot`.
struct PipeItem {
  int bh, q0, kt0, kt1, slot;
};

// Stream-K schedule (persistent workgroups).  The work of a call is laid out
// as one sequence of units, a unit being one 64-key tile of one query tile of
// 64*tu rows (128 with the pair-split layout, 256 without): head by head,
// and within a head the query tiles in zigzag order 0, nqt-1, 1, nqt-2, ...
// (under the causal mask tile t needs min(tu(t+1), nkt) key tiles, so
// neighbours in this order pair short and long tiles).  Each tile is preceded
// by `lead` units that hold no work: they stand for the fixed cost of a
// piece (loading Q and the first K/V tiles, writing the result), so that
// chunks balance time rather than key tiles.  Chunk c of G holds units
// [b(c), b(c+1)) with b(c) = floor(c*T/G); each workgroup runs one chunk.
// A chunk is a list of pieces (a query tile's key range, or part of it); a
// piece that covers its whole tile writes O and L, any other writes a
// partial result to workspace slot 2c (the chunk's first piece) or 2c + 1
// (its last), and fa_merge_stream combines the pieces of each cut tile.
struct StreamPlan {
  long long T;         // units in the call
  long long per_head;  // units per head
  long long cq;        // T / G
  int cr;              // T % G
  int G;               // chunks = workgroups, 1 <= G <= min(T, kMaxChunks)
  int nqt, nkt;        // query tiles (64*tu rows), key tiles (64 keys)
  int tu;              // key tiles per query tile on the causal diagonal: 2 or 4
  int lead;            // empty units before each tile
  int tail;            // empty units after each tile
};

// Lead units of a tile: about a piece's fixed cost (loading Q and the first
// K/V tiles, the end-of-piece barriers and stores) in key tiles of its
// layout; timed per piece on MI355X at about 14k cycles for D = 128 against
// 2.3k per 128-row key tile (4.5k per 256-row one), 7.5k against 3k for
// D = 64.  Throughput is flat within a few units of these values; 0 (no
// lead) loses up to 20% on small causal problems.
constexpr int stream_lead(int D, bool pair) { return D == 128 ? (pair ? 5 : 4) : 6; }
// The same for the variable-length schedule, whose tiles are shorter (a
// sequence's last tile is often partly empty, and more pieces per chunk end
// early): measured with the pair-split layout on 32768 tokens in 32 (8)
// sequences, D = 128 causal, lead 7 against 5: 47.9 -> 45.3 us (93.7 ->
// 92.1); 9: 45.9 (92.3); 3: 52.8 (93.0).
constexpr int varlen_lead(int D, bool pair) { return pair ? 7 : stream_lead(D, pair); }
// Tail units of a causal tile: the extra cost of its diagonal key tiles
// (the last tu, partly masked; a wave whose rows end early waits for the
// others at each of them).  A per-workgroup timing fit at the headline
// shape (time = 1.8k + 2.2k per key tile + 14.4k per piece + 3.7k per
// diagonal key tile, cycles) suggested lead 3 and tail 4 for the pair-split
// layout; measured, that was within noise of lead 5 and tail 0 and 3%
// slower on B4 N2048, so no tail is used.
constexpr int stream_tail(int, bool) { return 0; }

// Key tiles of query tile t.
FA_HD inline int tile_w(int t, int nkt, int tu, bool causal) {
  return causal ? (tu * (t + 1) < nkt ? tu * (t + 1) : nkt) : nkt;
}

// Units of query tiles 0..t-1.
FA_HD inline long long prefix_nat(int t, int nkt, int tu, bool causal) {
  if (!causal) return (long long)t * nkt;
  const int a = nkt / tu;  // tiles i < a have tu*(i+1) <= nkt key tiles
  if (t <= a) return (long long)tu * t * (t + 1) / 2;
  return (long long)tu * a * (a + 1) / 2 + (long long)(t - a) * nkt;
}

// Layout of the stream schedule's kernel at D = 128: the pair-split 128-row
// tiles when there are fewer 256-row tiles than compute units and each
// compute unit's share is small (under 64 units of 128 rows by 64 keys), or
// when a non-causal call has at most one 128-row tile per compute unit (no
// tile is then cut); otherwise 256-row tiles, which move half the K/V bytes
// into LDS per MFMA.  Measured on MI355X (B x N, D = 128, units per compute
// unit), pair-split against 256-row: causal B8 N4096 (33) +2.6%, B4 N2048
// (4) +17%, non-causal B8 N4096 (64) +9%; causal B1 N16384 (64) -1.4%, B4
// N8192 (65) -0.5%, B2 N16384 (129) -5.6%, B1 N24576 (145) -8%, B1 N32768
// (257) -7%.  D = 64 and 32 always take 256-row tiles: their blocks are
// shorter, so sharing the per-step costs between two blocks matters more.
inline bool stream_pair(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, bool causal, int cus) {
  if (D != 128 || BH * ((Nq + kGridRows - 1) / kGridRows) >= (int64_t)cus) return false;
  const int64_t nqt = (Nq + kPairRows - 1) / kPairRows;
  const int nkt = (int)((Nk + kKeys - 1) / kKeys);
  if (!causal && BH * nqt <= (int64_t)cus) return true;
  return BH * prefix_nat((int)nqt, nkt, kPairRows / kKeys, causal) < 64LL * cus;
}

// Query tile at zigzag position o, and units of positions 0..o-1 (their key
// tiles and lead units).
FA_HD inline int zz_tile(int o, int nqt) {
  return (o & 1) ? nqt - 1 - (o >> 1) : (o >> 1);
}
FA_HD inline long long zz_prefix(int o, int nqt, int nkt, int tu, int lead,
                                               bool causal) {
  return prefix_nat((o + 1) >> 1, nkt, tu, causal) +
         (prefix_nat(nqt, nkt, tu, causal) - prefix_nat(nqt - (o >> 1), nkt, tu, causal)) +
         (long long)lead * o;
}

// Zigzag position of the tile holding head-relative unit r (0 <= r < per_head).
FA_HD inline int zz_find(long long r, int nqt, int nkt, int tu, int lead,
                                       bool causal) {
  int lo = 0, hi = nqt - 1;  // zz_prefix(lo) <= r always holds
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (zz_prefix(mid, nqt, nkt, tu, lead, causal) <= r)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// floor(c * T / G), without 64-bit division (c * cr < G^2 < 2^32).
FA_HD inline long long chunk_start(const StreamPlan &sp, int c) {
  return (long long)c * sp.cq + (long long)((uint32_t)c * (uint32_t)sp.cr / (uint32_t)sp.G);
}

// The pieces of chunk ch, in order: next() yields each piece that holds key
// tiles (a chunk may also cover lead units only) as a PipeItem with query
// tile index t (rows t*64*tu ...).
struct ChunkWalk {
  long long left;  // units of the chunk not walked yet
  int ch, bh, zo, u;
  bool first;

  FA_HD void init(const StreamPlan &sp, int chunk, bool causal) {
    ch = chunk;
    const long long u0 = chunk_start(sp, ch);
    left = chunk_start(sp, ch + 1) - u0;
    // position of the chunk's first unit: head, zigzag tile position, unit
    // within the tile's lead units and key tiles
    bh = (int)(u0 / sp.per_head);
    const long long r0 = u0 - (long long)bh * sp.per_head;
    zo = zz_find(r0, sp.nqt, sp.nkt, sp.tu, sp.lead + sp.tail, causal);
    u = (int)(r0 - zz_prefix(zo, sp.nqt, sp.nkt, sp.tu, sp.lead + sp.tail, causal));
    first = true;
  }
  // The same start, read from the host's table (ChunkStarts).
  FA_HD void init_at(const StreamPlan &sp, int chunk, uint32_t w0, uint32_t w1) {
    ch = chunk;
    left = chunk_start(sp, ch + 1) - chunk_start(sp, ch);
    bh = (int)(w0 & 0xffffu);
    zo = (int)(w0 >> 16);
    u = (int)w1;
    first = true;
  }

  FA_HD bool next(const StreamPlan &sp, bool causal, PipeItem &it, int &t) {
    const int E = sp.lead;
    while (left > 0) {
      t = zz_tile(zo, sp.nqt);
      const int w = tile_w(t, sp.nkt, sp.tu, causal);
      const int span = E + w + sp.tail;
      const int u1 = left < (long long)(span - u) ? u + (int)left : span;
      const int kt0 = u <= E ? 0 : (u - E < w ? u - E : w);
      const int kt1 = u1 <= E ? 0 : (u1 - E < w ? u1 - E : w);
      left -= u1 - u;
      u = 0;  // the next piece starts a tile
      const int bh_t = bh;
      if (++zo == sp.nqt) {
        zo = 0;
        ++bh;
      }
      if (kt1 > kt0) {
        it.bh = bh_t;
        it.kt0 = kt0;
        it.kt1 = kt1;
        it.slot = (kt0 == 0 && kt1 == w) ? -1 : 2 * ch + (first ? 0 : 1);
        first = false;
        return true;
      }
    }
    return false;
  }
};

// The query tile holding the first unit of chunk j, and whether boundary j
// cuts it (lies after its first key tile, with no earlier boundary doing
// so).  Its pieces: chunk j-1 (its first piece when it starts at the tile,
// in its lead units or in the previous tile's tail units, else its last),
// then every chunk c >= j that starts before the tile's last key tile ends
// (its first piece).
struct CutTile {
  long long sl0, s0, s1;  // the tile's lead units, first key tile, end
  long long bprev;        // first unit of chunk j-1
  int bh, t, j;
  bool cut;

  FA_HD void init(const StreamPlan &sp, int jj, bool causal) {
    j = jj;
    const long long bj = chunk_start(sp, j);
    bh = (int)(bj / sp.per_head);
    const long long base = (long long)bh * sp.per_head;
    const int zo = zz_find(bj - base, sp.nqt, sp.nkt, sp.tu, sp.lead + sp.tail, causal);
    t = zz_tile(zo, sp.nqt);
    sl0 = base + zz_prefix(zo, sp.nqt, sp.nkt, sp.tu, sp.lead + sp.tail, causal);
    s0 = sl0 + sp.lead;
    s1 = s0 + tile_w(t, sp.nkt, sp.tu, causal);
    bprev = chunk_start(sp, j - 1);
    cut = bj > s0 && bj < s1 && bprev <= s0;
  }
  // Workspace slot of the tile's piece in chunk cc (cc = j-1, j, j+1, ...),
  // -1 past its last piece.
  FA_HD int slot(const StreamPlan &sp, int cc) const {
    if (cc >= sp.G || (cc >= j && chunk_start(sp, cc) >= s1)) return -1;
    // chunk j-1 holds key tiles of an earlier tile (this one is then its
    // last piece) iff it starts before the end of the previous tile's key
    // tiles, tail units before this tile's lead
    return (cc == j - 1 && bprev < sl0 - sp.tail) ? 2 * cc + 1 : 2 * cc;
  }
};

// At most this many chunks (workgroups) per call: the host's tables below
// are kernel arguments.
constexpr int kMaxChunks = 256;

// Where each chunk's walk starts (ChunkWalk::init: head, zigzag position,
// unit within the tile), and the cut tiles with their pieces (CutTile),
// computed on the host in one pass over the unit sequence and passed to the
// kernels as arguments: on the device, ChunkWalk::init costs a 64-bit
// division and a binary search per workgroup (about 1.7 us at the
// kernel's start, measured on MI355X), and CutTile::init the same per
// combining workgroup.
struct ChunkStarts {
  uint32_t w[2 * kMaxChunks];  // chunk c: bh | zo << 16, u
};
// Cut i: w[2i] = bh | t << 16; w[2i+1] = j | pieces << 16 | odd << 31,
// where j is the first chunk boundary strictly inside the tile's key tiles,
// the pieces are those of chunks j-1, j, ..., j+pieces-2, with workspace
// slots 2(j-1) + odd (odd: chunk j-1 holds key tiles of an earlier tile, so
// this is its last piece) and 2c for c >= j (their first pieces).
struct CutList {
  int n;
  uint32_t w[2 * (kMaxChunks - 1)];
};
FA_HD inline int cut_slot(uint32_t w1, int k) {
  const int j = (int)(w1 & 0xffffu);
  return k == 0 ? 2 * (j - 1) + (int)(w1 >> 31) : 2 * (j - 1 + k);
}
FA_HD inline int cut_pieces(uint32_t w1) { return (int)((w1 >> 16) & 0x7fffu); }

// Stream-K schedule of the pipelined kernel (16-bit inputs): one
// chunk per compute unit.  With four or more 128-row query tiles per compute
// unit the longest-first grid of fa_fwd already keeps every unit busy to the
// end, and a chunk would hold many pieces, each paying its own prologue: the
// call then takes that grid.  Returns false for the paths that take no
// workspace.
// A plan over query tiles of qt rows (a multiple of kKeys) with `lead` and
// `tail` units of fixed cost per tile, dealt to at most min(cus,
// kMaxChunks) chunks; the tables limit BH and the query tiles to 16 bits.
inline bool plan_rows(int64_t BH, int64_t Nq, int64_t Nk, int64_t qt, int lead, int tail,
                      bool causal, int cus, StreamPlan &sp) {
  if (cus < 1 || BH > 0xffff || (Nq + qt - 1) / qt > 0xffff) return false;
  const int nkt = (int)((Nk + kKeys - 1) / kKeys);
  const int nqt = (int)((Nq + qt - 1) / qt);
  sp.tu = (int)(qt / kKeys);
  sp.nqt = nqt;
  sp.nkt = nkt;
  sp.lead = lead;
  sp.tail = tail;
  sp.per_head = prefix_nat(nqt, nkt, sp.tu, causal) + (long long)(sp.lead + sp.tail) * nqt;
  sp.T = BH * sp.per_head;
  const int gmax = cus < kMaxChunks ? cus : kMaxChunks;
  sp.G = (int)(sp.T < gmax ? sp.T : gmax);
  sp.cq = sp.T / sp.G;
  sp.cr = (int)(sp.T % sp.G);
  return true;
}

inline bool make_plan(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, int dtype, bool causal,
               int cus, StreamPlan &sp, size_t &ws_bytes) {
  ws_bytes = 0;
  if (dtype == FA_F32 || cus < 1) return false;
  const int64_t pair_rows = kPairRows;
  if (BH * ((Nq + pair_rows - 1) / pair_rows) >= 4 * (int64_t)cus) return false;
  // the tables hold head and tile indices in 16 bits
  if (BH > 0xffff || (Nq + pair_rows - 1) / pair_rows > 0xffff) return false;
  const bool pair = stream_pair(BH, Nq, Nk, D, causal, cus);
  const int64_t qt = pair ? pair_rows : kGridRows;
  plan_rows(BH, Nq, Nk, qt, stream_lead((int)D, pair),
            causal ? stream_tail((int)D, pair) : 0, causal, cus, sp);
  ws_bytes = (size_t)2 * sp.G * qt * (size_t)(D + 4) * 4;
  return true;
}

// Key chunks of a variable-length query tile with nkt (>= 1) key tiles when
// a split allows at most NC chunks of at least KC key tiles: a chunk length
// kc = ceil(nkt / min(NC, ceil(nkt / KC))) and ceil(nkt / kc) chunks (returned,
// kc written).  Counting the chunks from kc rather than taking
// min(NC, ceil(nkt / KC)) itself keeps every chunk non-empty: capping the
// count at NC lengthens the chunks, and the rounded-up length can then cover
// the tile in fewer of them (nkt = 129, NC = 16, KC = 8: kc = 9, 15 chunks).
FA_HD inline int varlen_split(int nkt, int NC, int KC, int &kc) {
  int n = (nkt + KC - 1) / KC;
  if (n > NC) n = NC;
  if (n < 1) n = 1;
  kc = (nkt + n - 1) / n;
  return (nkt + kc - 1) / kc;
}

// The tables of a plan, in one pass over its tiles (heads in order, each
// head's tiles in zigzag order), with the chunk boundaries b(c) =
// chunk_start(c) advancing alongside: chunk c starts in the tile whose units
// [lead start, end of tail) hold b(c); a tile is cut iff some boundary j
// lies strictly inside its key tiles (s0 < b(j) < s1), the first such j
// naming it (as CutTile).  The same as ChunkWalk::init and CutTile for
// every chunk and boundary (checked on the host over many plans).
inline void make_tables(const StreamPlan &sp, bool causal, ChunkStarts &cs, CutList &cl) {
  const long long BH = sp.T / sp.per_head;
  int c = 0;   // next chunk start to place
  int jj = 0;  // first boundary after the current tile's first key tile
  long long base = 0;
  cl.n = 0;
  for (long long bh = 0; bh < BH; ++bh)
    for (int zo = 0; zo < sp.nqt; ++zo) {
      const int t = zz_tile(zo, sp.nqt);
      const long long s0 = base + sp.lead;
      const long long s1 = s0 + tile_w(t, sp.nkt, sp.tu, causal);
      const long long end = s1 + sp.tail;
      for (; c < sp.G && chunk_start(sp, c) < end; ++c) {
        cs.w[2 * c] = (uint32_t)bh | ((uint32_t)zo << 16);
        cs.w[2 * c + 1] = (uint32_t)(chunk_start(sp, c) - base);
      }
      while (jj < sp.G && chunk_start(sp, jj) <= s0) ++jj;
      if (jj >= 1 && jj < sp.G && chunk_start(sp, jj) < s1) {
        int pieces = 1;
        for (int cc = jj; cc < sp.G && chunk_start(sp, cc) < s1; ++cc) ++pieces;
        const bool odd = chunk_start(sp, jj - 1) < base - sp.tail;
        cl.w[2 * cl.n] = (uint32_t)bh | ((uint32_t)t << 16);
        cl.w[2 * cl.n + 1] = (uint32_t)jj | ((uint32_t)pieces << 16) | (odd ? 1u << 31 : 0u);
        ++cl.n;
      }
      base = end;
    }
}


}  // namespace fa_sched
