// kvc_ring_capi.cpp -- host-only C entry points over the ring planner
// (kvc_ring.hpp), built without HIP so the index arithmetic of the cache can
// be exercised and fuzzed on a CPU-only machine.
#include <cstdint>
#include <string>
#include <vector>

#include "kvc_ring.hpp"
#include "kvc_tiles.hpp"

namespace {
thread_local std::string g_ring_err;
}

extern "C" {

void* kvr_new(int32_t frame_seqlen, int32_t sink_tok, int32_t win_tok) {
  auto* st = new kvc::RingState();
  st->init(frame_seqlen, sink_tok, win_tok);
  return st;
}

void kvr_free(void* p) { delete static_cast<kvc::RingState*>(p); }

const char* kvr_error(void) { return g_ring_err.c_str(); }

// Returns the number of segments written to segs[4*i .. 4*i+3] = (region, dst, src, n), or -1.
int32_t kvr_append(void* p, int32_t n_frames, int32_t t0, int32_t replace, int32_t* segs, int32_t max_segs) {
  auto* st = static_cast<kvc::RingState*>(p);
  std::vector<kvc::Seg> s;
  int64_t g0 = 0;
  kvc::RingState nx = *st;
  if (!kvc::plan_append(nx, n_frames, t0, replace != 0, &s, &g0, &g_ring_err)) return -1;
  if ((int32_t)s.size() > max_segs) { g_ring_err = "too many segments"; return -1; }
  *st = nx;
  for (size_t i = 0; i < s.size(); ++i) {
    segs[4 * i] = s[i].region; segs[4 * i + 1] = s[i].dst; segs[4 * i + 2] = s[i].src; segs[4 * i + 3] = s[i].n;
  }
  return (int32_t)s.size();
}

int32_t kvr_sink_push(void* p, int32_t n_frames, int32_t bank_tok0, int32_t t0) {
  auto* st = static_cast<kvc::RingState*>(p);
  std::vector<kvc::Seg> s;
  return kvc::plan_sink_push(*st, n_frames, bank_tok0, t0, &s, &g_ring_err) ? (int32_t)s.size() : -1;
}

int32_t kvr_retime(void* p, int32_t delta, int32_t clamp0, int32_t lo, int32_t hi) {
  auto* st = static_cast<kvc::RingState*>(p);
  std::vector<kvc::Range> r;
  return kvc::plan_retime(*st, delta, clamp0 != 0, lo, hi, &r, &g_ring_err) ? (int32_t)r.size() : -1;
}

int32_t kvr_compact(void* p, const int32_t* keep, int32_t n) {
  auto* st = static_cast<kvc::RingState*>(p);
  std::vector<int32_t> src;
  return kvc::plan_compact(*st, keep, n, &src, &g_ring_err) ? (int32_t)src.size() : -1;
}

// counters: [n_valid, ns, hs, nw, hw, win_buf, newest_valid, newest_frames]
void kvr_counters(void* p, int64_t* out) {
  auto* st = static_cast<kvc::RingState*>(p);
  out[0] = st->n_valid(); out[1] = st->ns; out[2] = st->hs; out[3] = st->nw; out[4] = st->hw;
  out[5] = st->win_buf; out[6] = st->newest_valid; out[7] = st->newest_frames; out[8] = st->global_end;
}

void kvr_logical(void* p, int32_t* t, int64_t* g) { static_cast<kvc::RingState*>(p)->logical_times(t, g); }

// physical (region, slot) of every logical entry
void kvr_physical(void* p, int32_t* region, int32_t* slot) {
  auto* st = static_cast<kvc::RingState*>(p);
  for (int32_t l = 0; l < st->n_valid(); ++l) st->phys(l, region + l, slot + l);
}

// The attention kernels' key-tile order (kvc_tiles.hpp), built for the host so
// that CPU tests can check it.  Visible slot ranges [lo0, n0) and [lo1, n1);
// an empty range 0 is replaced by range 1, as the attention launch does.
// kvr_tile_count returns the number of tiles.  kvr_tile_order writes
// (tile << 1) | range of tiles first .. first + count - 1 of the sequence
// (edges_last: whole tiles first, else logical order) to out, the same from
// the whole-tile lookup the pipelined steps use to out_whole, and returns how
// many of them come before the first edge tile; -1 for a bad range.
static kvc::KeyRegions tile_ranges(int32_t lo0, int32_t n0, int32_t lo1, int32_t n1) {
  kvc::KeyRegions k{};
  k.lo[0] = lo0;
  k.n[0] = n0;
  k.lo[1] = lo1;
  k.n[1] = n1;
  if (kvc::range_tiles(k, 0) == 0) {
    k.lo[0] = lo1;
    k.n[0] = n1;
    k.lo[1] = 0;
    k.n[1] = 0;
  }
  return k;
}

int32_t kvr_tile_count(int32_t lo0, int32_t n0, int32_t lo1, int32_t n1) {
  const kvc::KeyRegions k = tile_ranges(lo0, n0, lo1, n1);
  return kvc::range_tiles(k, 0) + kvc::range_tiles(k, 1);
}

int32_t kvr_tile_order(int32_t lo0, int32_t n0, int32_t lo1, int32_t n1, int32_t edges_last, int32_t first,
                       int32_t count, int32_t* out, int32_t* out_whole) {
  const kvc::KeyRegions k = tile_ranges(lo0, n0, lo1, n1);
  const int nt0 = kvc::range_tiles(k, 0), nt = nt0 + kvc::range_tiles(k, 1);
  if (first < 0 || count < 0 || first + count > nt) return -1;
  kvc::TileSeq s = edges_last ? kvc::tile_seq_edges_last(k, nt0, nt) : kvc::tile_seq(k, nt0, nt);
  s.first = first;
  for (int32_t it = 0; it < count; ++it) {
    out[it] = s.at(it);
    out_whole[it] = (s.base_w(it) / kvc::kBN) << 1 | s.region_w(it);
  }
  return s.whole_prefix(count);
}

// the key-part count of a split attention launch with `total` workgroups over `ntiles` key tiles
int32_t kvr_split_parts(int32_t total, int32_t ntiles) { return kvc::split_parts(total, ntiles); }

int32_t kvr_causal_clean_steps(int32_t n0, int32_t n1, int32_t ntile0, int32_t nt, int32_t lim_lo) {
  return kvc::causal_clean_steps(n0, n1, ntile0, nt, lim_lo);
}

}  // extern "C"
