// kvc_ring.hpp -- host-side index arithmetic of the bounded video KV cache.
//
// Pure C++ (no HIP): the same code drives libkvc and a host-only test build.
//
// The cache has two physical regions:
//   sink   -- S_tok slots; filled by the first S_tok tokens ever appended and
//             then pinned (LingBot-World 2.0 article, "sink_size attention
//             sink"); a FIFO of blocks only under the Rolling-Sink push.
//   window -- W_tok slots used as a ring: appending past capacity advances the
//             head over the oldest tokens.  This is the eviction rule of the
//             LingBot-World 2.0 article, section "how the window rolls when
//             full" (evict as many of the oldest non-sink tokens as the new
//             block overflows the capacity by), done as a ring-head advance
//             instead of a left shift of everything after the sink.
// Logical order (what exports, retime ranges, scores and keep lists use):
// sink oldest..newest, then window oldest..newest.
//
// Invariants kept by every operation below:
//   * sink_filled < S_tok  implies sink_head == 0 and window_filled == 0;
//   * window_filled < W_tok implies window_head == 0;
// so the valid physical slots are always the prefixes [0, sink_filled) and
// [0, window_filled) of the two regions.
#pragma once

#include <algorithm>
#include <cstdint>
#include <string>
#include <vector>

namespace kvc {

constexpr int32_t kMaxPos = 16383;

enum RegionId : int32_t { kSink = 0, kWin = 1 };

// A run of n consecutive tokens of the source (starting at token `src`) that
// lands on n consecutive physical slots of a region (starting at `dst`).
struct Seg {
  int32_t region;
  int32_t dst;
  int32_t src;
  int32_t n;
};

// A run of n consecutive physical slots of one region.
struct Range {
  int32_t region;
  int32_t lo;
  int32_t n;
};

struct RingState {
  int32_t S = 1;          // tokens per frame
  int32_t S_tok = 0;      // sink capacity
  int32_t W_tok = 0;      // window capacity
  int32_t ns = 0, hs = 0; // sink filled / head
  int32_t nw = 0, hw = 0; // window filled / head
  int32_t win_buf = 0;    // current window buffer (0/1)
  int64_t global_end = 0;
  bool newest_valid = false;
  int32_t newest_frames = 0;
  int32_t newest_n = 0;
  int64_t newest_g = 0;
  std::vector<Seg> newest_segs;
  // host mirrors, per physical slot of the current buffers
  std::vector<int32_t> t_sink, t_win;
  std::vector<int64_t> g_sink, g_win;

  void init(int32_t frame_seqlen, int32_t sink_tok, int32_t win_tok) {
    S = frame_seqlen;
    S_tok = sink_tok;
    W_tok = win_tok;
    ns = hs = nw = hw = win_buf = 0;
    global_end = 0;
    newest_valid = false;
    newest_segs.clear();
    t_sink.assign(S_tok, 0);
    g_sink.assign(S_tok, 0);
    t_win.assign(W_tok, 0);
    g_win.assign(W_tok, 0);
  }

  int32_t n_valid() const { return ns + nw; }

  // logical index -> (region, physical slot)
  void phys(int32_t l, int32_t* region, int32_t* slot) const {
    if (l < ns) {
      *region = kSink;
      *slot = (hs + l) % S_tok;
    } else {
      *region = kWin;
      *slot = (hw + (l - ns)) % W_tok;
    }
  }

  int32_t t_at(int32_t region, int32_t slot) const { return region == kSink ? t_sink[slot] : t_win[slot]; }
  int64_t g_at(int32_t region, int32_t slot) const { return region == kSink ? g_sink[slot] : g_win[slot]; }

  void logical_times(int32_t* t, int64_t* g) const {
    for (int32_t l = 0; l < n_valid(); ++l) {
      int32_t r, s;
      phys(l, &r, &s);
      if (t) t[l] = t_at(r, s);
      if (g) g[l] = g_at(r, s);
    }
  }

  // Physical ranges covering logical [lo, hi) (at most two per region).
  std::vector<Range> ranges(int32_t lo, int32_t hi) const {
    std::vector<Range> out;
    auto add = [&](int32_t region, int32_t cap, int32_t head, int32_t a, int32_t b) {
      if (b <= a) return;
      int32_t p = (head + a) % cap;
      int32_t n = b - a;
      int32_t first = std::min(n, cap - p);
      out.push_back({region, p, first});
      if (n > first) out.push_back({region, 0, n - first});
    };
    add(kSink, S_tok, hs, std::max(lo, 0), std::min(hi, ns));
    add(kWin, W_tok, hw, std::max(lo, ns) - ns, std::max(hi, ns) - ns);
    return out;
  }

  void write_mirror(const std::vector<Seg>& segs, int32_t t0, int64_t g0, bool set_g) {
    for (const Seg& s : segs)
      for (int32_t i = 0; i < s.n; ++i) {
        int32_t tok = s.src + i;
        int32_t t = t0 + tok / S;
        if (s.region == kSink) {
          t_sink[s.dst + i] = t;
          if (set_g) g_sink[s.dst + i] = g0 + tok;
        } else {
          t_win[s.dst + i] = t;
          if (set_g) g_win[s.dst + i] = g0 + tok;
        }
      }
  }

  // Recompute where the newest chunk's tokens live from the g mirrors; it
  // stays addressable only if all of its tokens are still cached.
  void rebuild_newest() {
    if (!newest_valid) return;
    struct Hit { int32_t region, slot, off; };
    std::vector<Hit> hits;
    for (int32_t l = 0; l < n_valid(); ++l) {
      int32_t r, s;
      phys(l, &r, &s);
      int64_t g = g_at(r, s);
      if (g >= newest_g && g < newest_g + newest_n) hits.push_back({r, s, (int32_t)(g - newest_g)});
    }
    if ((int32_t)hits.size() != newest_n) {
      newest_valid = false;
      newest_segs.clear();
      return;
    }
    std::sort(hits.begin(), hits.end(), [](const Hit& a, const Hit& b) { return a.off < b.off; });
    newest_segs.clear();
    for (const Hit& h : hits) {
      if (!newest_segs.empty()) {
        Seg& b = newest_segs.back();
        if (b.region == h.region && b.dst + b.n == h.slot && b.src + b.n == h.off) {
          ++b.n;
          continue;
        }
      }
      newest_segs.push_back({h.region, h.slot, h.off, 1});
    }
  }
};

// Plan an append of n_frames frames (N = n_frames * S tokens) at time t0.
// On success fills `segs` and updates `st` (mirrors included); on failure
// leaves `st` untouched and returns false with a message.
inline bool plan_append(RingState& st, int32_t n_frames, int32_t t0, bool replace, std::vector<Seg>* segs,
                        int64_t* g0_out, std::string* err) {
  const int64_t N64 = (int64_t)n_frames * st.S;
  if (n_frames <= 0) { *err = "n_frames must be positive"; return false; }
  if (N64 > st.W_tok) { *err = "chunk larger than the rolling window"; return false; }
  if (t0 < -kMaxPos || (int64_t)t0 + n_frames - 1 > kMaxPos) { *err = "time index out of range"; return false; }
  const int32_t N = (int32_t)N64;
  segs->clear();
  if (replace) {
    if (!st.newest_valid) { *err = "no newest chunk to replace"; return false; }
    if (st.newest_frames != n_frames) { *err = "replace: frame count differs from the newest chunk"; return false; }
    *segs = st.newest_segs;
    *g0_out = st.newest_g;
    st.write_mirror(*segs, t0, 0, false);
    return true;
  }
  RingState nx = st;
  int32_t n_s = 0;
  if (nx.ns < nx.S_tok) {
    n_s = std::min(N, nx.S_tok - nx.ns);
    segs->push_back({kSink, nx.ns, 0, n_s});   // sink head is 0 while filling
    nx.ns += n_s;
  }
  int32_t n_w = N - n_s;
  if (n_w > 0) {
    if (nx.nw + n_w > nx.W_tok) {            // evict the oldest window tokens: advance the head
      int32_t e = nx.nw + n_w - nx.W_tok;
      nx.hw = (nx.hw + e) % nx.W_tok;
      nx.nw -= e;
    }
    int32_t pos = (nx.hw + nx.nw) % nx.W_tok;
    int32_t first = std::min(n_w, nx.W_tok - pos);
    segs->push_back({kWin, pos, n_s, first});
    if (n_w > first) segs->push_back({kWin, 0, n_s + first, n_w - first});
    nx.nw += n_w;
  }
  *g0_out = nx.global_end;
  nx.write_mirror(*segs, t0, nx.global_end, true);
  nx.newest_valid = true;
  nx.newest_frames = n_frames;
  nx.newest_n = N;
  nx.newest_g = nx.global_end;
  nx.newest_segs = *segs;
  nx.global_end += N;
  st = std::move(nx);
  return true;
}

// Rolling-Sink push: overwrite the oldest N sink slots with bank tokens
// [bank_tok0, bank_tok0 + N) at times t0 + token/S.
inline bool plan_sink_push(RingState& st, int32_t n_frames, int32_t bank_tok0, int32_t t0, std::vector<Seg>* segs,
                           std::string* err) {
  const int64_t N64 = (int64_t)n_frames * st.S;
  if (n_frames <= 0) { *err = "n_frames must be positive"; return false; }
  if (st.S_tok == 0 || st.ns != st.S_tok) { *err = "sink_push needs a full sink"; return false; }
  if (N64 > st.S_tok) { *err = "sink_push block larger than the sink"; return false; }
  if (t0 < -kMaxPos || (int64_t)t0 + n_frames - 1 > kMaxPos) { *err = "time index out of range"; return false; }
  const int32_t N = (int32_t)N64;
  RingState nx = st;
  segs->clear();
  int32_t first = std::min(N, nx.S_tok - nx.hs);
  segs->push_back({kSink, nx.hs, 0, first});
  if (N > first) segs->push_back({kSink, 0, first, N - first});
  nx.hs = (nx.hs + N) % nx.S_tok;
  nx.write_mirror(*segs, t0, bank_tok0, true);
  nx.rebuild_newest();
  st = std::move(nx);
  return true;
}

// Plan a retime of logical [lo, hi).  Returns the physical ranges.
inline bool plan_retime(RingState& st, int32_t delta, bool clamp0, int32_t lo, int32_t hi, std::vector<Range>* rs,
                        std::string* err) {
  if (lo < 0 || hi > st.n_valid() || lo > hi) { *err = "retime range outside [0, n_valid)"; return false; }
  if (delta < -kMaxPos || delta > kMaxPos) { *err = "retime delta out of range"; return false; }
  *rs = st.ranges(lo, hi);
  for (const Range& r : *rs)
    for (int32_t i = 0; i < r.n; ++i) {
      int64_t t = st.t_at(r.region, r.lo + i);
      int64_t tn = clamp0 ? std::max<int64_t>(0, t + delta) : t + delta;
      if (tn < -kMaxPos || tn > kMaxPos) { *err = "retime moves a time index out of range"; return false; }
    }
  for (const Range& r : *rs)
    for (int32_t i = 0; i < r.n; ++i) {
      int32_t& t = r.region == kSink ? st.t_sink[r.lo + i] : st.t_win[r.lo + i];
      t = clamp0 ? std::max(0, t + delta) : t + delta;
    }
  return true;
}

// Plan a compaction: validates keep[], returns the source physical window
// slot of each kept window entry (packed to [0, n) of the other buffer).
inline bool plan_compact(RingState& st, const int32_t* keep, int32_t n_keep, std::vector<int32_t>* src_win,
                         std::string* err) {
  const int32_t n = st.n_valid();
  if (n_keep <= 0 || keep == nullptr) { *err = "keep_idx empty"; return false; }
  for (int32_t i = 0; i < n_keep; ++i) {
    if (keep[i] < 0 || keep[i] >= n) { *err = "keep_idx out of range"; return false; }
    if (i > 0 && keep[i] <= keep[i - 1]) { *err = "keep_idx not sorted and unique"; return false; }
  }
  if (n_keep < st.ns) { *err = "keep_idx drops a sink entry"; return false; }
  for (int32_t i = 0; i < st.ns; ++i)
    if (keep[i] != i) { *err = "keep_idx drops a sink entry"; return false; }
  src_win->clear();
  for (int32_t i = st.ns; i < n_keep; ++i) src_win->push_back((st.hw + (keep[i] - st.ns)) % st.W_tok);
  RingState nx = st;
  std::vector<int32_t> t2(nx.W_tok, 0);
  std::vector<int64_t> g2(nx.W_tok, 0);
  for (size_t j = 0; j < src_win->size(); ++j) {
    t2[j] = st.t_win[(*src_win)[j]];
    g2[j] = st.g_win[(*src_win)[j]];
  }
  nx.t_win.swap(t2);
  nx.g_win.swap(g2);
  nx.nw = (int32_t)src_win->size();
  nx.hw = 0;
  nx.win_buf ^= 1;
  nx.rebuild_newest();
  st = std::move(nx);
  return true;
}

}  // namespace kvc
