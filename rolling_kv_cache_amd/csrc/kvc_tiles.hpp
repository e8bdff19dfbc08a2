// kvc_tiles.hpp -- the order in which the attention kernels visit key tiles,
// shared by the HIP kernels and a host-only build that tests it on the CPU.
#pragma once

#include "kvc_device.hpp"

#if defined(__HIPCC__)
#define KVC_HD __host__ __device__ __forceinline__
#else
#define KVC_HD inline
#endif

namespace kvc {

constexpr int kBN = 64;   // keys per tile

KVC_HD int imin(int a, int b) { return a < b ? a : b; }
KVC_HD int imax(int a, int b) { return a > b ? a : b; }

// a (bit = 0) or b (bit = 1), by arithmetic on a bit the optimizer cannot see
// through: a select between two fields of a struct on a computed bit becomes a
// load from a computed address, which keeps the struct in scratch memory.
KVC_HD int pick(int bit, int a, int b) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm("" : "+v"(bit));
#endif
  return a + bit * (b - a);
}

// Key tiles in visiting order.  Logical order: the tiles covering region 0's
// visible slots [lo0, n0), then region 1's.  Edges-last order (any order
// gives the same softmax when no row's keys depend on the order, i.e. without
// a causal limit): each range's whole tiles first, then its edge tiles -- the
// first tile when the range starts inside it, the last when it ends inside it
// -- so all but the last few tiles need no mask.  base = first slot of the
// tile (64-aligned), valid = slots of the tile before the range end, lead =
// slots of the tile before the range start.  `first` shifts the sequence (a
// split-key workgroup starts at its part's first tile).
struct TileSeq {
  int ntile0, ntiles;
  int t00, t01;            // first tile of each range
  int lo0, lo1, n0, n1;
  int first;
  int f0, f1;              // tiles visited first from each range (all of them in logical order)
  int w00, w01;            // the first of those in each range
  int epos;                // edge tiles visited after them: 2 bits each, in order, naming range 0's
                           // first (0) or last (1) tile, or range 1's first (2) or last (3)
  int t0last, t1last;      // last tile of each range
  // range and first slot of the it-th tile, for a tile visited before the edges (any tile in logical
  // order): two plain selects, which stay branch-free inside the pipelined step
  KVC_HD int region_w(int it) const { return it + first < f0 ? 0 : 1; }
  KVC_HD int base_w(int it) const {
    const int jt = it + first;
    return (jt < f0 ? w00 + jt : w01 + jt - f0) * kBN;
  }
  KVC_HD int valid_w(int it) const { return (it + first < f0 ? n0 : n1) - base_w(it); }
  KVC_HD int lead_w(int it) const { return (it + first < f0 ? lo0 : lo1) - base_w(it); }
  // (tile index << 1) | range of any tile of the sequence
  KVC_HD int at(int it) const {
    const int jt = it + first;
    if (jt < f0 + f1) return (base_w(it) / kBN) << 1 | region_w(it);
    const int b = (epos >> (2 * (jt - f0 - f1))) & 3;
    const int r = b >> 1;
    const int te = pick(b & 1, pick(r, t00, t01), pick(r, t0last, t1last));
    return (te << 1) | r;
  }
  KVC_HD int region(int it) const { return at(it) & 1; }
  KVC_HD int base(int it) const { return (at(it) >> 1) * kBN; }
  KVC_HD int valid(int it) const {
    const int x = at(it);
    return pick(x & 1, n0, n1) - (x >> 1) * kBN;
  }
  KVC_HD int lead(int it) const {
    const int x = at(it);
    return pick(x & 1, lo0, lo1) - (x >> 1) * kBN;
  }
  // tiles of the sequence, counted from `first`, that need no mask (edges-last order)
  KVC_HD int whole_prefix(int n) const { return imax(0, imin(n, f0 + f1 - first)); }
};

KVC_HD TileSeq tile_seq(const KeyRegions& k, int ntile0, int ntiles) {
  TileSeq s{};
  s.ntile0 = ntile0;
  s.ntiles = ntiles;
  s.t00 = k.lo[0] / kBN;
  s.t01 = k.lo[1] / kBN;
  s.lo0 = k.lo[0];
  s.lo1 = k.lo[1];
  s.n0 = k.n[0];
  s.n1 = k.n[1];
  s.f0 = ntile0;
  s.f1 = ntiles - ntile0;
  s.w00 = s.t00;
  s.w01 = s.t01;
  s.t0last = s.t00 + ntile0 - 1;
  s.t1last = s.t01 + ntiles - ntile0 - 1;
  return s;
}

KVC_HD TileSeq tile_seq_edges_last(const KeyRegions& k, int ntile0, int ntiles) {
  TileSeq s = tile_seq(k, ntile0, ntiles);
  const int nt1 = ntiles - ntile0;
  // a range's first tile is an edge when the range starts inside it, its last when it ends inside it
  const int e0lo = ntile0 > 0 && s.lo0 % kBN != 0;
  const int e0hi = ntile0 > 0 && s.n0 % kBN != 0 && !(ntile0 == 1 && e0lo);
  const int e1lo = nt1 > 0 && s.lo1 % kBN != 0;
  const int e1hi = nt1 > 0 && s.n1 % kBN != 0 && !(nt1 == 1 && e1lo);
  s.w00 = s.t00 + e0lo;
  s.f0 = ntile0 - e0lo - e0hi;
  s.w01 = s.t01 + e1lo;
  s.f1 = nt1 - e1lo - e1hi;
  s.t0last = s.t00 + ntile0 - 1;
  s.t1last = s.t01 + nt1 - 1;
  int ne = 0;
  if (e0lo) s.epos |= 0 << (2 * ne++);
  if (e0hi) s.epos |= 1 << (2 * ne++);
  if (e1lo) s.epos |= 2 << (2 * ne++);
  if (e1hi) s.epos |= 3 << (2 * ne++);
  return s;
}

// tiles covering region r's visible slots
KVC_HD int range_tiles(const KeyRegions& k, int r) {
  return k.n[r] > k.lo[r] ? (k.n[r] + kBN - 1) / kBN - k.lo[r] / kBN : 0;
}

// Block-causal (logical order, both ranges from slot 0): the number of tiles
// from tile 1 on that are whole and end before lim_lo -- the key count every
// row of the block sees -- capped at nt - 1.  In closed form: region 0's
// tiles below n0 / 64 and lim_lo / 64, then, when all of region 0's tiles
// 1 .. ntile0 - 1 qualify, region 1's below n1 / 64 and (lim_lo - n0) / 64.
KVC_HD int causal_clean_steps(int n0, int n1, int ntile0, int nt, int lim_lo) {
  const int w0 = imin(n0 / kBN, lim_lo / kBN);
  const int c = (ntile0 > 1 && w0 < ntile0) ? w0 - 1
                                            : ntile0 - 1 + (lim_lo >= n0 ? imin(n1 / kBN, (lim_lo - n0) / kBN) : 0);
  return imax(0, imin(c, nt - 1));
}

// key parts for a split launch (one workgroup per CU at a time): the count in
// 2..8 whose workgroups fill the last round of 256 CUs best, when that beats
// the unsplit launch's fill by more than 2 % (ties: fewer parts), with at
// least four tiles per part and kSplitRows rows of partials (the split
// buffers' size: kparts * workgroups * 256 rows never exceeds it); 1 = no
// split.  Host code.
inline int split_parts(int total, int ntiles) {
  auto fill = [](int wgs) { return (double)wgs / (256.0 * ((wgs + 255) / 256)); };
  int best = 1;
  double best_fill = fill(total);
  for (int kp = 2; kp <= 8; ++kp) {
    if (kp * 4 > ntiles || (int64_t)kp * total * 256 > kSplitRows) break;
    const double f = fill(kp * total);
    if (f > best_fill + 0.02) {
      best = kp;
      best_fill = f;
    }
  }
  return best;
}

}  // namespace kvc
