// kvc_host.cpp -- the C ABI of libkvc: validation, ring planning, workspace
// layout, RoPE tables and kernel launches.  No device memory is allocated here:
// the caller provides the workspace (and the score scratch).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "kvc.h"
#include "kvc_device.hpp"
#include "kvc_launch.hpp"
#include "kvc_ring.hpp"

static_assert(KVC_MAX_POS == kvc::kMaxPos, "time table range");
static_assert(KVC_RELAX_NOALLOC_SCRATCH_BYTES == kvc::kRelaxNoallocScratch, "relax scratch size");
static_assert(KVC_PATH_RUNNING_MAX == kvc::kPathRunningMax && KVC_PATH_GENERAL == kvc::kPathGeneral &&
                  KVC_PATH_NO_SPLIT == kvc::kPathNoSplit,
              "path bits");

namespace {

thread_local std::string g_err;

kvc_status fail(kvc_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int32_t round64(int32_t x) { return (x + kvc::kTile - 1) / kvc::kTile * kvc::kTile; }

struct RegionLayout {
  size_t ka, kb, v, t, g;
};

struct Layout {
  bool ok = false;
  int32_t S_tok = 0, W_tok = 0, SP = 0, WP = 0, bank_tok = 0;
  int32_t D = 0, DA = 0, DB = 0, dt = 0, bw = 0, esz = 0;
  RegionLayout sink{}, win[2]{};
  size_t bank_k = 0, bank_v = 0, tab_t = 0, tab_h = 0, tab_w = 0, keep = 0, att_flags = 0, total = 0;
  size_t mem_k = 0, mem_v = 0, split_o = 0, split_ml = 0;
  size_t placed_sink = 0, placed_win = 0;   // raw keys: time band placed for the matrix-core attention
};

Layout make_layout(int32_t sink_frames, int32_t window_frames, int32_t S, int32_t H, int32_t D, kvc_dtype dt,
                   int32_t bank_frames, uint32_t cflags) {
  Layout L;
  if (sink_frames < 0 || window_frames < 1 || S < 1 || H < 1 || bank_frames < 0) return L;
  if (D != 64 && D != 128) return L;
  if (dt != KVC_BF16 && dt != KVC_F32) return L;
  const int64_t s_tok = (int64_t)sink_frames * S, w_tok = (int64_t)window_frames * S;
  const int64_t b_tok = (int64_t)bank_frames * S;
  if (s_tok + w_tok > (1 << 26) || b_tok > (1 << 26) || H > 4096) return L;
  L.S_tok = (int32_t)s_tok;
  L.W_tok = (int32_t)w_tok;
  // memory tokens (MemRoPE) live in 2S extra sink-region slots after the sink
  L.SP = round64(L.S_tok + ((cflags & KVC_CREATE_MEMORY) ? 2 * S : 0));
  L.WP = round64(L.W_tok);
  L.bank_tok = (int32_t)b_tok;
  L.D = D;
  L.esz = dt == KVC_BF16 ? 2 : 4;
  L.bw = 2 * (D / 6);
  L.dt = D - 2 * L.bw;
  const int32_t E = 16 / L.esz;
  L.DA = (L.dt + E - 1) / E * E;
  L.DB = D - L.DA;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  auto region = [&](int32_t cap) {
    RegionLayout r;
    r.ka = take((size_t)H * cap * L.DA * L.esz);
    r.kb = take((size_t)H * cap * L.DB * L.esz);
    r.v = take((size_t)H * cap * D * L.esz);
    r.t = take((size_t)cap * 4);
    r.g = take((size_t)cap * 8);
    return r;
  };
  L.sink = region(L.SP);
  L.win[0] = region(L.WP);
  if (cflags & KVC_CREATE_COMPACT) L.win[1] = region(L.WP);
  L.bank_k = take((size_t)H * L.bank_tok * D * L.esz);
  L.bank_v = take((size_t)H * L.bank_tok * D * L.esz);
  L.tab_t = take((size_t)(2 * KVC_MAX_POS + 1) * (L.dt / 2) * 2 * 4);
  L.tab_h = take((size_t)S * (L.bw / 2) * 2 * 4);
  L.tab_w = take((size_t)S * (L.bw / 2) * 2 * 4);
  L.keep = take((size_t)L.WP * 4);
  // one recompute flag per 256-query attention block of the largest query chunk, and with split keys
  // per (block, part): kparts * blocks * 256 <= kSplitRows bounds those units
  size_t n_flags = (size_t)H * (((size_t)KVC_MAX_Q_FRAMES * S + 255) / 256);
  if (cflags & KVC_CREATE_SPLIT_ATTEND) n_flags = std::max(n_flags, (size_t)kvc::kSplitRows / 256);
  L.att_flags = take(n_flags * 4);
  if (cflags & KVC_CREATE_SPLIT_ATTEND) {
    L.split_o = take((size_t)kvc::kSplitRows * 128 * 4);
    L.split_ml = take((size_t)kvc::kSplitRows * 2 * 4);
  }
  if (cflags & KVC_CREATE_MEMORY) {
    L.mem_k = take((size_t)2 * H * S * D * 4);
    L.mem_v = take((size_t)2 * H * S * D * 4);
  }
  // raw-key caches on the matrix-core paths (bf16, head_dim 128 or 64): KA planes with every slot's time
  // band placed at its current time, written once per attend call and read by the plain attention kernels
  if ((cflags & KVC_CREATE_RAW_KEYS) && L.esz == 2 && (D == 128 || D == 64)) {
    L.placed_sink = take((size_t)H * L.SP * L.DA * L.esz);
    L.placed_win = take((size_t)H * L.WP * L.DA * L.esz);
  }
  L.total = off;
  L.ok = true;
  return L;
}

}  // namespace

struct kvc_cache {
  int32_t sink_frames, window_frames, S, H, D, grid_w, grid_h, bank_frames;
  kvc_dtype dt;
  uint32_t cflags;
  Layout L;
  char* ws;
  kvc::Geo geo;
  kvc::Tables tab;
  kvc::RegionPtrs sink, win[2];
  void* bank_k;
  void* bank_v;
  int32_t* keep_dev;
  int32_t* att_flags;
  int32_t* keep_pinned;      // two halves of WP entries: the host fills one while the other may still be read
  int32_t* keep_pinned_dev;  // the same memory's device-visible address
  hipEvent_t keep_evt[2];    // recorded after the staging kernel that reads each half
  bool keep_pending[2];
  int32_t keep_half;
  hipEvent_t order_evt;      // kvc_set_stream: the new stream waits for the old one's queued work
  hipStream_t stream;
  uint32_t paths;            // kPath* bits (kvc_set_paths)
  kvc::RingState st;
  bool poisoned;
  float mem_alpha[2];
  int32_t mem_frames;       // frames folded into the memories so far
  int32_t max_keys;         // > 0: attention reads only the newest max_keys entries
  const void* group;        // layer group (kvc_create_group): shared tag, layer index, stride
  int32_t layer;
  int64_t layer_stride;
  // row statistics (kvc_attend_stats -> kvc_score_with_stats): epoch counts the calls that changed the
  // entries or what attention reads; the latest statistics are valid only while it stays where it was
  uint64_t epoch;
  bool stats_valid;
  uint64_t stats_epoch;
  const float* stats_buf;
  int32_t stats_frames, stats_t0;
};

namespace {

kvc::RegionPtrs region_ptrs(char* ws, const RegionLayout& r, int32_t cap) {
  kvc::RegionPtrs p;
  p.ka = ws + r.ka;
  p.kb = ws + r.kb;
  p.v = ws + r.v;
  p.t = (int32_t*)(ws + r.t);
  p.g = (int64_t*)(ws + r.g);
  p.cap = cap;
  return p;
}

kvc_status check(kvc_handle h) {
  if (!h) return fail(KVC_EINVAL, "null handle");
  if (h->poisoned) return fail(KVC_ESTATE, "handle poisoned by an earlier device error");
  return KVC_OK;
}

kvc_status device_result(kvc_handle h, hipError_t e, const char* what) {
  if (e == hipSuccess) return KVC_OK;
  h->poisoned = true;
  return fail(KVC_EDEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

// The window region the cache currently reads from.
const kvc::RegionPtrs& cur_win(kvc_handle h) { return h->win[h->st.win_buf]; }

kvc::KeyRegions key_regions(kvc_handle h) {
  kvc::KeyRegions k{};
  const kvc::RegionPtrs& w = cur_win(h);
  k.ka[0] = h->sink.ka;
  k.kb[0] = h->sink.kb;
  k.v[0] = h->sink.v;
  k.t[0] = h->sink.t;
  k.cap[0] = h->sink.cap;
  k.n[0] = h->st.ns;
  k.ka[1] = w.ka;
  k.kb[1] = w.kb;
  k.v[1] = w.v;
  k.t[1] = w.t;
  k.cap[1] = w.cap;
  k.n[1] = h->st.nw;
  return k;
}

// Launch the append kernel over a list of segments (in batches of kMaxSegs).
hipError_t launch_segments(kvc_handle h, const std::vector<kvc::Seg>& segs, const void* k, const void* v,
                           int64_t k_tok, int64_t k_head, int64_t v_tok, int64_t v_head, int32_t t0, int64_t g0,
                           int32_t bank_lo, int32_t bank_hi, int32_t layers = 1, int64_t layer_stride = 0,
                           int64_t src_stride = 0) {
  for (size_t b = 0; b < segs.size(); b += kvc::kMaxSegs) {
    kvc::AppendArgs a{};
    a.layers = layers;
    a.layer_stride = layer_stride;
    a.src_stride = src_stride;
    a.time_raw = (h->cflags & KVC_CREATE_RAW_KEYS) ? 1 : 0;
    a.k = k;
    a.v = v;
    a.k_tok = k_tok;
    a.k_head = k_head;
    a.v_tok = v_tok;
    a.v_head = v_head;
    a.reg[0] = h->sink;
    a.reg[1] = cur_win(h);
    int32_t ns = 0;
    for (size_t i = b; i < segs.size() && ns < kvc::kMaxSegs; ++i, ++ns) {
      const kvc::Seg& s = segs[i];
      kvc::SegW& w = a.seg[ns];
      w.region = s.region;
      w.dst = s.dst;
      w.src = s.src;
      w.n = s.n;
    }
    a.nseg = ns;
    a.t0 = t0;
    a.g0 = g0;
    a.bank_k = h->bank_k;
    a.bank_v = h->bank_v;
    a.bank_tok = h->L.bank_tok;
    a.bank_lo = bank_lo;
    a.bank_hi = bank_hi;
    a.geo = h->geo;
    a.tab = h->tab;
    hipError_t e = kvc::launch_append(a, h->stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

void build_tables(int32_t D, int32_t S, int32_t grid_w, std::vector<float>* tt, std::vector<float>* th,
                  std::vector<float>* tw) {
  const int32_t bw = 2 * (D / 6), dt = D - 2 * bw;
  const int32_t Pt = dt / 2, Pb = bw / 2;
  auto theta = [](int32_t j, int32_t width) { return std::pow(10000.0, -(2.0 * j) / (double)width); };
  tt->assign((size_t)(2 * KVC_MAX_POS + 1) * Pt * 2, 0.f);
  for (int32_t p = -KVC_MAX_POS; p <= KVC_MAX_POS; ++p)
    for (int32_t j = 0; j < Pt; ++j) {
      const double ang = (double)p * theta(j, dt);
      float* o = &(*tt)[((size_t)(p + KVC_MAX_POS) * Pt + j) * 2];
      o[0] = (float)std::cos(ang);
      o[1] = (float)std::sin(ang);
    }
  const int32_t grid_h = S / grid_w;
  th->assign((size_t)S * Pb * 2, 0.f);
  tw->assign((size_t)S * Pb * 2, 0.f);
  for (int32_t p = 0; p < grid_h; ++p)
    for (int32_t j = 0; j < Pb; ++j) {
      const double ang = (double)p * theta(j, bw);
      (*th)[((size_t)p * Pb + j) * 2] = (float)std::cos(ang);
      (*th)[((size_t)p * Pb + j) * 2 + 1] = (float)std::sin(ang);
    }
  for (int32_t p = 0; p < grid_w; ++p)
    for (int32_t j = 0; j < Pb; ++j) {
      const double ang = (double)p * theta(j, bw);
      (*tw)[((size_t)p * Pb + j) * 2] = (float)std::cos(ang);
      (*tw)[((size_t)p * Pb + j) * 2 + 1] = (float)std::sin(ang);
    }
}

// Raw-key caches: scores and Relax scores read the keys as attention sees them, so their scratch gets
// a copy of the KA planes with each slot's time band rotated to its current time.
size_t placed_ka_bytes(kvc_handle h) {
  if (!(h->cflags & KVC_CREATE_RAW_KEYS)) return 0;
  return align_up((size_t)h->H * h->L.SP * h->L.DA * h->geo.esz) + align_up((size_t)h->H * h->L.WP * h->L.DA * h->geo.esz);
}

hipError_t launch_placed_ka(kvc_handle h, char* dst, kvc::KeyRegions* keys) {
  kvc::RetimeArgs a{};
  a.reg[0] = h->sink;
  a.reg[1] = cur_win(h);
  a.out_ka[0] = dst;
  a.out_ka[1] = dst + align_up((size_t)h->H * h->L.SP * h->L.DA * h->geo.esz);
  const int32_t n[2] = {h->st.ns, h->st.nw};
  int32_t blocks = 0;
  for (int r = 0; r < 2; ++r) {
    if (n[r] == 0) continue;
    a.rng[a.nrng].region = r;
    a.rng[a.nrng].lo = 0;
    a.rng[a.nrng].n = n[r];
    a.rng[a.nrng].blk0 = blocks;
    blocks += (n[r] + kvc::retime_slots(h->H, h->geo.D, h->geo.esz) - 1) / kvc::retime_slots(h->H, h->geo.D, h->geo.esz);
    ++a.nrng;
  }
  a.keys = 1;
  a.geo = h->geo;
  a.tab = h->tab;
  keys->ka[0] = a.out_ka[0];
  keys->ka[1] = a.out_ka[1];
  return kvc::launch_retime(a, blocks, h->stream);
}

// Raw-key caches on the matrix-core path: place the time band of every slot the attention may read --
// the valid prefixes of the sink and the current window, and the memory frames at their times -- into
// the workspace's placed KA planes in one pass, and point the key regions' KA planes there, so that the
// plain kernels run (each staged tile would otherwise be rotated again by every query block).  Slots
// past the valid prefixes keep what the placed planes held (zeros from creation, or keys placed by an
// earlier call): finite, and masked by the attention.
hipError_t launch_placed_attend(kvc_handle h, kvc::AttendArgs& a) {
  char* ps = h->ws + h->L.placed_sink;
  char* pw = h->ws + h->L.placed_win;
  kvc::RetimeArgs r{};
  r.reg[0] = h->sink;
  r.reg[1] = cur_win(h);
  r.out_ka[0] = ps;
  r.out_ka[1] = pw;
  int32_t blocks = 0;
  auto add = [&](int32_t region, int32_t lo, int32_t n, int32_t fixed, int32_t t) {
    if (n <= 0) return;
    kvc::RangeW& g = r.rng[r.nrng++];
    g.region = region;
    g.lo = lo;
    g.n = n;
    g.blk0 = blocks;
    g.fixed = fixed;
    g.tfix = t;
    blocks += (n + kvc::retime_slots(h->H, h->geo.D, h->geo.esz) - 1) / kvc::retime_slots(h->H, h->geo.D, h->geo.esz);
  };
  add(kvc::kSink, 0, h->st.ns, 0, 0);
  add(kvc::kWin, 0, h->st.nw, 0, 0);
  if (a.mem_lo != INT32_MAX) {
    add(kvc::kSink, a.mem_lo, h->S, 1, a.mem_t[0]);
    add(kvc::kSink, a.mem_lo + h->S, h->S, 1, a.mem_t[1]);
  }
  r.keys = 1;
  r.geo = h->geo;
  r.tab = h->tab;
  for (int i = 0; i < 2; ++i) {
    if (a.keys.ka[i] == h->sink.ka)
      a.keys.ka[i] = ps;
    else if (a.keys.ka[i] == cur_win(h).ka)
      a.keys.ka[i] = pw;
  }
  a.raw = 0;
  a.mem_lo = INT32_MAX;
  return kvc::launch_retime(r, blocks, h->stream);
}

bool same_ring(const kvc::RingState& a, const kvc::RingState& b) {
  return a.ns == b.ns && a.hs == b.hs && a.nw == b.nw && a.hw == b.hw && a.win_buf == b.win_buf &&
         a.global_end == b.global_end && a.newest_valid == b.newest_valid && a.newest_frames == b.newest_frames &&
         a.t_sink == b.t_sink && a.t_win == b.t_win && a.g_sink == b.g_sink && a.g_win == b.g_win;
}

// A batched call takes consecutive layers of one group, all in the same state and on the same stream; a
// single-layer call is the set {h}.
kvc_status check_layers(const kvc_handle* hs, int32_t n) {
  if (!hs || n < 1) return fail(KVC_EINVAL, "empty layer set");
  for (int32_t i = 0; i < n; ++i)
    if (kvc_status s = check(hs[i])) return s;
  for (int32_t i = 1; i < n; ++i) {
    if (!hs[0]->group || hs[i]->group != hs[0]->group || hs[i]->layer != hs[0]->layer + i)
      return fail(KVC_EINVAL, "layers must be consecutive members of one kvc_create_group group");
    if (hs[i]->stream != hs[0]->stream) return fail(KVC_EINVAL, "layers must share a stream");
    if (!same_ring(hs[i]->st, hs[0]->st)) return fail(KVC_ESTATE, "layers are not in the same cache state");
  }
  return KVC_OK;
}

kvc_status device_result_layers(const kvc_handle* hs, int32_t n, hipError_t e, const char* what) {
  if (e == hipSuccess) return KVC_OK;
  for (int32_t i = 0; i < n; ++i) hs[i]->poisoned = true;
  return fail(KVC_EDEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

extern "C" {

size_t kvc_workspace_bytes(int32_t sink_frames, int32_t window_frames, int32_t frame_seqlen, int32_t heads,
                           int32_t head_dim, kvc_dtype dt, int32_t bank_frames, uint32_t create_flags) {
  Layout L = make_layout(sink_frames, window_frames, frame_seqlen, heads, head_dim, dt, bank_frames, create_flags);
  return L.ok ? L.total : 0;
}

kvc_status kvc_create(int32_t sink_frames, int32_t window_frames, int32_t frame_seqlen, int32_t heads,
                      int32_t head_dim, int32_t grid_w, kvc_dtype dt, int32_t bank_frames, uint32_t create_flags,
                      void* workspace, size_t ws_bytes, void* hip_stream, kvc_handle* out) {
  if (!out) return fail(KVC_EINVAL, "out is null");
  *out = nullptr;
  Layout L = make_layout(sink_frames, window_frames, frame_seqlen, heads, head_dim, dt, bank_frames, create_flags);
  if (!L.ok) return fail(KVC_EINVAL, "unsupported geometry (head_dim must be 64 or 128; sizes positive)");
  if (grid_w < 1 || frame_seqlen % grid_w != 0) return fail(KVC_EINVAL, "frame_seqlen must be a multiple of grid_w");
  if (create_flags & ~(KVC_CREATE_COMPACT | KVC_CREATE_RAW_KEYS | KVC_CREATE_MEMORY | KVC_CREATE_SPLIT_ATTEND))
    return fail(KVC_EINVAL, "unknown create flag");
  if ((create_flags & KVC_CREATE_MEMORY) && !(create_flags & KVC_CREATE_RAW_KEYS))
    return fail(KVC_EINVAL, "memory tokens need KVC_CREATE_RAW_KEYS");
  if ((create_flags & KVC_CREATE_RAW_KEYS) && !(dt == KVC_BF16 || dt == KVC_F32))
    return fail(KVC_EINVAL, "raw keys need a bf16 or fp32 cache");
  if (!workspace) return fail(KVC_EINVAL, "workspace is null");
  if ((uintptr_t)workspace % kAlign != 0) return fail(KVC_EINVAL, "workspace must be 256-byte aligned");
  if (ws_bytes < L.total) return fail(KVC_ENOMEM, "workspace smaller than kvc_workspace_bytes()");
  kvc_cache* h = new (std::nothrow) kvc_cache();
  if (!h) return fail(KVC_ENOMEM, "host allocation failed");
  h->sink_frames = sink_frames;
  h->window_frames = window_frames;
  h->S = frame_seqlen;
  h->H = heads;
  h->D = head_dim;
  h->grid_w = grid_w;
  h->grid_h = frame_seqlen / grid_w;
  h->bank_frames = bank_frames;
  h->dt = dt;
  h->cflags = create_flags;
  h->L = L;
  h->ws = (char*)workspace;
  h->stream = (hipStream_t)hip_stream;
  h->poisoned = false;
  h->geo = kvc::Geo{heads, head_dim, frame_seqlen, grid_w, L.DA, L.DB, L.dt, L.bw, L.esz};
  h->tab = kvc::Tables{(const float*)(h->ws + L.tab_t), (const float*)(h->ws + L.tab_h),
                       (const float*)(h->ws + L.tab_w), KVC_MAX_POS};
  h->sink = region_ptrs(h->ws, L.sink, L.SP);
  h->win[0] = region_ptrs(h->ws, L.win[0], L.WP);
  h->win[1] = (create_flags & KVC_CREATE_COMPACT) ? region_ptrs(h->ws, L.win[1], L.WP) : h->win[0];
  h->bank_k = h->ws + L.bank_k;
  h->bank_v = h->ws + L.bank_v;
  h->keep_dev = (int32_t*)(h->ws + L.keep);
  h->att_flags = (int32_t*)(h->ws + L.att_flags);
  h->keep_pinned = nullptr;
  h->keep_pinned_dev = nullptr;
  h->keep_pending[0] = h->keep_pending[1] = false;
  h->keep_half = 0;
  h->paths = 0;
  h->max_keys = 0;
  h->group = nullptr;
  h->layer = 0;
  h->layer_stride = 0;
  h->mem_alpha[0] = 0.9f;
  h->mem_alpha[1] = 0.5f;
  h->mem_frames = 0;
  h->st.init(frame_seqlen, L.S_tok, L.W_tok);
  hipError_t e = hipEventCreateWithFlags(&h->order_evt, hipEventDisableTiming);
  if (e != hipSuccess) {
    delete h;
    return fail(KVC_ENOMEM, std::string("event: ") + hipGetErrorString(e));
  }
  if (create_flags & KVC_CREATE_COMPACT) {
    int n_evt = 0;
    e = hipHostMalloc((void**)&h->keep_pinned, (size_t)2 * L.WP * 4, hipHostMallocMapped | hipHostMallocCoherent);
    if (e == hipSuccess) e = hipHostGetDevicePointer((void**)&h->keep_pinned_dev, h->keep_pinned, 0);
    for (; e == hipSuccess && n_evt < 2; ++n_evt) e = hipEventCreateWithFlags(&h->keep_evt[n_evt], hipEventDisableTiming);
    if (e != hipSuccess) {
      for (int i = 0; i < n_evt; ++i) (void)hipEventDestroy(h->keep_evt[i]);
      if (h->keep_pinned) (void)hipHostFree(h->keep_pinned);
      (void)hipEventDestroy(h->order_evt);
      delete h;
      return fail(KVC_ENOMEM, std::string("pinned staging: ") + hipGetErrorString(e));
    }
  }
  std::vector<float> tt, th, tw;
  build_tables(head_dim, frame_seqlen, grid_w, &tt, &th, &tw);
  e = kvc::launch_fill_zero(h->ws, L.total, h->stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h->ws + L.tab_t, tt.data(), tt.size() * 4, hipMemcpyHostToDevice, h->stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h->ws + L.tab_h, th.data(), th.size() * 4, hipMemcpyHostToDevice, h->stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h->ws + L.tab_w, tw.data(), tw.size() * 4, hipMemcpyHostToDevice, h->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) {
    if (h->keep_pinned) {
      (void)hipHostFree(h->keep_pinned);
      (void)hipEventDestroy(h->keep_evt[0]);
      (void)hipEventDestroy(h->keep_evt[1]);
    }
    (void)hipEventDestroy(h->order_evt);
    delete h;
    return fail(KVC_EDEVICE, std::string("create: ") + hipGetErrorString(e));
  }
  *out = h;
  return KVC_OK;
}

size_t kvc_group_workspace_bytes(int32_t n_layers, int32_t sink_frames, int32_t window_frames,
                                 int32_t frame_seqlen, int32_t heads, int32_t head_dim, kvc_dtype dt,
                                 int32_t bank_frames, uint32_t create_flags) {
  if (n_layers < 1) return 0;
  const size_t one = kvc_workspace_bytes(sink_frames, window_frames, frame_seqlen, heads, head_dim, dt, bank_frames,
                                         create_flags);
  return one * (size_t)n_layers;
}

kvc_status kvc_create_group(int32_t n_layers, int32_t sink_frames, int32_t window_frames, int32_t frame_seqlen,
                            int32_t heads, int32_t head_dim, int32_t grid_w, kvc_dtype dt, int32_t bank_frames,
                            uint32_t create_flags, void* workspace, size_t ws_bytes, void* hip_stream,
                            kvc_handle* out) {
  if (!out || n_layers < 1) return fail(KVC_EINVAL, "out is null or n_layers < 1");
  const size_t one = kvc_workspace_bytes(sink_frames, window_frames, frame_seqlen, heads, head_dim, dt, bank_frames,
                                         create_flags);
  if (one == 0) return fail(KVC_EINVAL, "unsupported geometry");
  if (ws_bytes < one * (size_t)n_layers) return fail(KVC_ENOMEM, "workspace smaller than kvc_group_workspace_bytes()");
  for (int32_t l = 0; l < n_layers; ++l) out[l] = nullptr;
  for (int32_t l = 0; l < n_layers; ++l) {
    kvc_status s = kvc_create(sink_frames, window_frames, frame_seqlen, heads, head_dim, grid_w, dt, bank_frames,
                              create_flags, (char*)workspace + one * l, one, hip_stream, &out[l]);
    if (s != KVC_OK) {
      const std::string msg = g_err;
      for (int32_t j = 0; j < l; ++j) {
        kvc_destroy(out[j]);
        out[j] = nullptr;
      }
      return fail(s, msg);
    }
    out[l]->group = workspace;
    out[l]->layer = l;
    out[l]->layer_stride = (int64_t)one;
  }
  return KVC_OK;
}

kvc_status kvc_destroy(kvc_handle h) {
  if (!h) return fail(KVC_EINVAL, "null handle");
  if (h->keep_pinned) {
    for (int i = 0; i < 2; ++i) {
      if (h->keep_pending[i]) (void)hipEventSynchronize(h->keep_evt[i]);
      (void)hipEventDestroy(h->keep_evt[i]);
    }
    (void)hipHostFree(h->keep_pinned);
  }
  (void)hipEventDestroy(h->order_evt);
  delete h;
  return KVC_OK;
}

kvc_status kvc_set_stream(kvc_handle h, void* hip_stream) {
  if (kvc_status s = check(h)) return s;
  const hipStream_t ns = (hipStream_t)hip_stream;
  if (ns != h->stream) {
    // work already queued on the old stream (which may read or write the workspace) comes first
    hipError_t e = hipEventRecord(h->order_evt, h->stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(ns, h->order_evt, 0);
    if (kvc_status s = device_result(h, e, "set_stream")) return s;
  }
  h->stream = ns;
  return KVC_OK;
}

kvc_status kvc_set_paths(kvc_handle h, uint32_t paths) {
  if (kvc_status s = check(h)) return s;
  if (paths & ~(KVC_PATH_RUNNING_MAX | KVC_PATH_GENERAL | KVC_PATH_NO_SPLIT)) return fail(KVC_EINVAL, "unknown path bit");
  h->paths = paths;
  return KVC_OK;
}

kvc_status kvc_append(kvc_handle h, const void* k, const void* v, int32_t n_frames, int32_t t_index,
                      uint32_t flags) {
  if (kvc_status s = check(h)) return s;
  if (!k || !v) return fail(KVC_EINVAL, "k/v null");
  if (flags & ~KVC_APPEND_REPLACE_NEWEST) return fail(KVC_EINVAL, "unknown append flag");
  const bool replace = (flags & KVC_APPEND_REPLACE_NEWEST) != 0;
  kvc::RingState nx = h->st;
  std::vector<kvc::Seg> segs;
  int64_t g0 = 0;
  std::string err;
  if (!kvc::plan_append(nx, n_frames, t_index, replace, &segs, &g0, &err)) return fail(KVC_EINVAL, err);
  const int32_t N = n_frames * h->S;
  int32_t bank_lo = 0, bank_hi = 0;
  if (h->L.bank_tok > 0 && g0 < h->L.bank_tok) bank_hi = (int32_t)std::min<int64_t>(N, h->L.bank_tok - g0);
  const int64_t HD = (int64_t)h->H * h->D;
  // MemRoPE: the frames this append evicts (the oldest window entries) fold into the memories first
  const int32_t evicted = replace ? 0 : h->st.n_valid() + N - nx.n_valid();
  hipError_t e = hipSuccess;
  if ((h->cflags & KVC_CREATE_MEMORY) && evicted > 0) {
    if (evicted % h->S != 0 || h->st.ns != h->L.S_tok) return fail(KVC_ESTATE, "memory folds whole frames");
    kvc::MemFoldArgs m{};
    m.win = cur_win(h);
    m.sink = h->sink;
    m.state_k = (float*)(h->ws + h->L.mem_k);
    m.state_v = (float*)(h->ws + h->L.mem_v);
    m.hw = h->st.hw;
    m.W_tok = h->st.W_tok;
    m.n_frames = evicted / h->S;
    m.init = h->mem_frames == 0 ? 1 : 0;
    m.mem_lo = h->L.S_tok;
    m.alpha[0] = h->mem_alpha[0];
    m.alpha[1] = h->mem_alpha[1];
    m.geo = h->geo;
    e = kvc::launch_mem_fold(m, h->stream);
  }
  // the window region read by the kernel must be the post-plan buffer (unchanged by append)
  if (e == hipSuccess) e = launch_segments(h, segs, k, v, HD, h->D, HD, h->D, t_index, g0, bank_lo, bank_hi);
  if (kvc_status s = device_result(h, e, "append")) return s;
  if (h->cflags & KVC_CREATE_MEMORY) h->mem_frames += evicted / h->S;
  h->st = std::move(nx);
  ++h->epoch;
  return KVC_OK;
}

// row_m (optional): also write each query row's log2 softmax normaliser, [heads][q_frames * S]; *t0_out
// receives the time query frame 0 was rotated at
static kvc_status attend_impl(kvc_handle h, const void* q, int32_t q_frames, int32_t q_t_index, void* out,
                              int32_t causal_block, float* row_m = nullptr, int32_t* t0_out = nullptr) {
  if (!q || !out) return fail(KVC_EINVAL, "q/out null");
  if (q_frames < 1 || q_frames > KVC_MAX_Q_FRAMES) return fail(KVC_EINVAL, "q_frames out of range");
  if (h->st.n_valid() == 0) return fail(KVC_ESTATE, "attend on an empty cache");
  int32_t t0 = q_t_index;
  if (q_t_index == KVC_T_NEWEST) {
    if (!h->st.newest_valid) return fail(KVC_ESTATE, "no newest chunk for KVC_T_NEWEST");
    const kvc::Seg& s0 = h->st.newest_segs.front();
    t0 = h->st.t_at(s0.region, s0.dst) - s0.src / h->S;
  }
  if (t0 < -KVC_MAX_POS || (int64_t)t0 + q_frames - 1 > KVC_MAX_POS) return fail(KVC_EINVAL, "q time out of range");
  if (row_m != nullptr) {
    // the statistics stand in for the rows pass of a score over the valid entries: attention must read
    // exactly those (no memory tokens, no attention limit)
    if ((h->cflags & KVC_CREATE_MEMORY) && h->mem_frames > 0)
      return fail(KVC_EUNSUPPORTED, "row statistics with memory tokens");
    if (h->max_keys > 0 && h->max_keys < h->st.n_valid())
      return fail(KVC_EUNSUPPORTED, "row statistics with an attention limit");
  }
  kvc::AttendArgs a{};
  a.q = q;
  a.out = out;
  a.row_m = row_m;
  a.Lq = q_frames * h->S;
  a.t0 = t0;
  a.keys = key_regions(h);
  a.geo = h->geo;
  a.tab = h->tab;
  a.scale = (float)(1.0 / std::sqrt((double)h->D));
  a.flags = h->att_flags;
  a.causal_block = causal_block;
  a.raw = (h->cflags & KVC_CREATE_RAW_KEYS) ? 1 : 0;
  a.mem_lo = INT32_MAX;
  if ((h->cflags & KVC_CREATE_SPLIT_ATTEND) && h->D == 128 && h->geo.esz == 2) {
    a.split_o = (float*)(h->ws + h->L.split_o);
    a.split_ml = (float*)(h->ws + h->L.split_ml);
  }
  const int32_t n_valid = h->st.n_valid();
  if (h->max_keys > 0 && h->max_keys < n_valid) {
    // only the newest max_keys entries in logical order: at most two physical ranges (a window suffix
    // that wraps, or a sink tail plus the whole window) when the sink ring has not rolled
    if (causal_block > 0) return fail(KVC_EUNSUPPORTED, "block-causal attention with an attention limit");
    if (h->cflags & KVC_CREATE_MEMORY) return fail(KVC_EUNSUPPORTED, "memory tokens with an attention limit");
    // per region: the whole valid prefix when all of it is visible (key order does not matter),
    // else the physical ranges of its visible logical suffix
    const int32_t lo = n_valid - h->max_keys, ns = h->st.ns;
    std::vector<kvc::Range> rs;
    if (lo < ns) {
      if (lo == 0)
        rs.push_back({kvc::kSink, 0, ns});
      else
        for (const kvc::Range& r : h->st.ranges(lo, ns)) rs.push_back(r);
    }
    if (n_valid > std::max(lo, ns)) {
      if (lo <= ns)
        rs.push_back({kvc::kWin, 0, h->st.nw});
      else
        for (const kvc::Range& r : h->st.ranges(lo, n_valid)) rs.push_back(r);
    }
    if (rs.size() > 2) return fail(KVC_EUNSUPPORTED, "attention limit over a rolled sink");
    kvc::KeyRegions k{};
    for (size_t i = 0; i < rs.size(); ++i) {
      const kvc::RegionPtrs& R = rs[i].region == kvc::kSink ? h->sink : cur_win(h);
      k.ka[i] = R.ka;
      k.kb[i] = R.kb;
      k.v[i] = R.v;
      k.t[i] = R.t;
      k.cap[i] = R.cap;
      k.lo[i] = rs[i].lo;
      k.n[i] = rs[i].lo + rs[i].n;
    }
    if (rs.size() == 1) {             // an empty second range over the same buffer
      k.ka[1] = k.ka[0];
      k.kb[1] = k.kb[0];
      k.v[1] = k.v[0];
      k.t[1] = k.t[0];
      k.cap[1] = k.cap[0];
    }
    a.keys = k;
  }
  if ((h->cflags & KVC_CREATE_MEMORY) && h->mem_frames > 0 && !(h->max_keys > 0 && h->max_keys < n_valid)) {
    // the memories sit right before the oldest window entry: long at t_w - 2, short at t_w - 1
    if (causal_block > 0) return fail(KVC_EUNSUPPORTED, "block-causal attention with memory tokens");
    const int32_t t_w = h->st.t_at(kvc::kWin, h->st.hw);
    if (t_w - 2 < -KVC_MAX_POS) return fail(KVC_EINVAL, "memory time out of range");
    a.mem_lo = h->L.S_tok;
    a.mem_t[0] = t_w - 2;
    a.mem_t[1] = t_w - 1;
    a.keys.n[0] = h->L.S_tok + 2 * h->S;
  }
  hipError_t e = hipSuccess;
  // raw keys on the matrix-core path: the time band placed once, then the plain kernels
  if (a.raw && h->L.placed_win != 0 && !(h->paths & KVC_PATH_GENERAL)) e = launch_placed_attend(h, a);
  if (e == hipSuccess) e = kvc::launch_attend(a, h->paths, h->stream);
  if (t0_out != nullptr) *t0_out = t0;
  return device_result(h, e, "attend");
}

kvc_status kvc_attend(kvc_handle h, const void* q, int32_t q_frames, int32_t q_t_index, void* out) {
  if (kvc_status s = check(h)) return s;
  return attend_impl(h, q, q_frames, q_t_index, out, 0);
}

kvc_status kvc_attend_stats(kvc_handle h, const void* q, int32_t q_frames, int32_t q_t_index, void* out,
                            float* row_stats) {
  if (kvc_status s = check(h)) return s;
  if (!row_stats) return fail(KVC_EINVAL, "row_stats null");
  h->stats_valid = false;
  int32_t t0 = 0;
  if (kvc_status s = attend_impl(h, q, q_frames, q_t_index, out, 0, row_stats, &t0)) return s;
  h->stats_valid = true;
  h->stats_epoch = h->epoch;
  h->stats_buf = row_stats;
  h->stats_frames = q_frames;
  h->stats_t0 = t0;
  return KVC_OK;
}

kvc_status kvc_attend_blockcausal(kvc_handle h, const void* q, int32_t q_frames, int32_t q_t_index,
                                  int32_t block_frames, void* out) {
  if (kvc_status s = check(h)) return s;
  if (block_frames < 1 || block_frames > KVC_MAX_Q_FRAMES) return fail(KVC_EINVAL, "block_frames out of range");
  if (h->cflags & KVC_CREATE_MEMORY) return fail(KVC_EUNSUPPORTED, "block-causal attention with memory tokens");
  // key prefixes are taken in logical order, which must coincide with slot order
  if (h->st.hs != 0 || h->st.hw != 0)
    return fail(KVC_EUNSUPPORTED, "block-causal attention needs an unrolled cache (sink and window heads at 0)");
  return attend_impl(h, q, q_frames, q_t_index, out, block_frames * h->S);
}

static kvc_status retime_layers(const kvc_handle* hs, int32_t nl, int32_t delta, int32_t clamp0, int32_t slot_lo,
                                int32_t slot_hi) {
  if (kvc_status s = check_layers(hs, nl)) return s;
  kvc_handle h = hs[0];
  kvc::RingState nx = h->st;
  std::vector<kvc::Range> rs;
  std::string err;
  if (!kvc::plan_retime(nx, delta, clamp0 != 0, slot_lo, slot_hi, &rs, &err)) return fail(KVC_EINVAL, err);
  kvc::RetimeArgs a{};
  a.layers = nl;
  a.layer_stride = h->layer_stride;
  a.reg[0] = h->sink;
  a.reg[1] = cur_win(h);
  int32_t blocks = 0;
  a.nrng = (int32_t)rs.size();
  for (size_t i = 0; i < rs.size(); ++i) {
    a.rng[i].region = rs[i].region;
    a.rng[i].lo = rs[i].lo;
    a.rng[i].n = rs[i].n;
    a.rng[i].blk0 = blocks;
    blocks += (rs[i].n + kvc::retime_slots(h->H, h->geo.D, h->geo.esz) - 1) / kvc::retime_slots(h->H, h->geo.D, h->geo.esz);
  }
  a.delta = delta;
  a.clamp0 = clamp0 != 0;
  a.keys = (h->cflags & KVC_CREATE_RAW_KEYS) ? 0 : 1;     // raw keys: only the time indices move
  a.geo = h->geo;
  a.tab = h->tab;
  hipError_t e = kvc::launch_retime(a, blocks, h->stream);
  if (kvc_status s = device_result_layers(hs, nl, e, "retime")) return s;
  for (int32_t i = 0; i < nl; ++i) {
    hs[i]->st = nx;
    ++hs[i]->epoch;
  }
  return KVC_OK;
}

kvc_status kvc_retime(kvc_handle h, int32_t delta, int32_t clamp0, int32_t slot_lo, int32_t slot_hi) {
  return retime_layers(&h, 1, delta, clamp0, slot_lo, slot_hi);
}

kvc_status kvc_retime_layers(const kvc_handle* layers, int32_t n_layers, int32_t delta, int32_t clamp0,
                             int32_t slot_lo, int32_t slot_hi) {
  return retime_layers(layers, n_layers, delta, clamp0, slot_lo, slot_hi);
}

size_t kvc_score_scratch_bytes(kvc_handle h, int32_t q_frames) {
  if (!h || q_frames < 1 || q_frames > KVC_MAX_Q_FRAMES) return 0;
  const size_t Nq = (size_t)q_frames * h->S;
  return align_up((size_t)h->H * Nq * h->D * 4) + 2 * align_up((size_t)h->H * Nq * 4) +
         align_up((size_t)h->H * (h->L.SP + h->L.WP) * 4) + align_up((size_t)h->H * ((Nq + 255) / 256) * 4) +
         placed_ka_bytes(h);
}

// row_stats (optional): the rows pass's normalisers, from the latest kvc_attend_stats of these queries
static kvc_status score_impl(kvc_handle h, const void* q_win, int32_t q_frames, const int32_t* q_t, float* scores,
                             void* scratch, size_t scratch_bytes, const float* row_stats) {
  if (kvc_status s = check(h)) return s;
  if (!q_win || !q_t || !scores || !scratch) return fail(KVC_EINVAL, "null argument");
  if (q_frames < 1 || q_frames > KVC_MAX_Q_FRAMES) return fail(KVC_EINVAL, "q_frames out of range");
  if (scratch_bytes < kvc_score_scratch_bytes(h, q_frames)) return fail(KVC_ENOMEM, "score scratch too small");
  if ((uintptr_t)scratch % kAlign != 0) return fail(KVC_EINVAL, "scratch must be 256-byte aligned");
  if (h->st.n_valid() == 0) return fail(KVC_ESTATE, "score on an empty cache");
  kvc::ScoreArgs a{};
  for (int32_t f = 0; f < q_frames; ++f) {
    if (q_t[f] < -KVC_MAX_POS || q_t[f] > KVC_MAX_POS) return fail(KVC_EINVAL, "q_t out of range");
    a.qt[f] = q_t[f];
  }
  if (row_stats != nullptr) {
    bool same = h->stats_valid && h->stats_epoch == h->epoch && h->stats_buf == row_stats &&
                h->stats_frames == q_frames;
    for (int32_t f = 0; same && f < q_frames; ++f) same = q_t[f] == h->stats_t0 + f;
    if (!same)
      return fail(KVC_ESTATE, "row_stats are not the latest kvc_attend_stats of these query frames and times over "
                              "the current cache");
  }
  const size_t Nq = (size_t)q_frames * h->S;
  char* p = (char*)scratch;
  a.qh = (float*)p;
  p += align_up((size_t)h->H * Nq * h->D * 4);
  a.m = (float*)p;
  p += align_up((size_t)h->H * Nq * 4);
  a.l = (float*)p;
  p += align_up((size_t)h->H * Nq * 4);
  a.part = (float*)p;
  p += align_up((size_t)h->H * (h->L.SP + h->L.WP) * 4);
  a.flags = (int32_t*)p;
  p += align_up((size_t)h->H * ((Nq + 255) / 256) * 4);
  if (row_stats != nullptr) {   // the columns pass reads the attention's normalisers in place
    a.m = const_cast<float*>(row_stats);
    a.rows_given = 1;
  }
  a.q = q_win;
  a.scores = scores;
  a.Nq = (int32_t)Nq;
  a.keys = key_regions(h);
  a.ns = h->st.ns;
  a.hs = h->st.hs;
  a.S_tok = std::max(1, h->st.S_tok);
  a.nw = h->st.nw;
  a.hw = h->st.hw;
  a.W_tok = h->st.W_tok;
  a.geo = h->geo;
  a.tab = h->tab;
  a.scale = (float)(1.0 / std::sqrt((double)h->D));
  hipError_t e = hipSuccess;
  if (h->cflags & KVC_CREATE_RAW_KEYS) e = launch_placed_ka(h, p, &a.keys);
  if (e == hipSuccess) e = kvc::launch_score(a, h->paths, h->stream);
  return device_result(h, e, "score");
}

kvc_status kvc_score(kvc_handle h, const void* q_win, int32_t q_frames, const int32_t* q_t, float* scores,
                     void* scratch, size_t scratch_bytes) {
  return score_impl(h, q_win, q_frames, q_t, scores, scratch, scratch_bytes, nullptr);
}

kvc_status kvc_score_with_stats(kvc_handle h, const void* q_win, int32_t q_frames, const int32_t* q_t,
                                const float* row_stats, float* scores, void* scratch, size_t scratch_bytes) {
  if (kvc_status s = check(h)) return s;
  if (!row_stats) return fail(KVC_EINVAL, "row_stats null");
  return score_impl(h, q_win, q_frames, q_t, scores, scratch, scratch_bytes, row_stats);
}

static int32_t relax_slices(kvc_handle h) { return (h->S + kvc::kRelaxSlice - 1) / kvc::kRelaxSlice; }

size_t kvc_relax_scratch_bytes(kvc_handle h) {
  if (!h) return 0;
  const size_t nf = (size_t)(h->st.S_tok + h->st.W_tok) / h->S;   // at most this many whole frames
  return align_up(nf * relax_slices(h) * h->H * h->D * 4) + align_up(nf * h->H * h->D * 4) +
         align_up((size_t)kvc::kRelaxMaxFrames * kvc::kRelaxMaxFrames * 4) + placed_ka_bytes(h);
}

// Relax Forcing scores on a given scratch (validated by the callers); `noalloc` only changes the error
// text for a scratch that is too small.
static kvc_status relax_impl(kvc_handle h, int32_t tail_frames, float weight, float* scores, void* scratch,
                             size_t scratch_bytes, bool noalloc) {
  if (!scores) return fail(KVC_EINVAL, "null argument");
  if (!(weight >= 0.f && weight <= 1.f)) return fail(KVC_EINVAL, "weight outside [0, 1]");
  if (scratch_bytes < kvc_relax_scratch_bytes(h))
    return fail(KVC_ENOMEM, noalloc ? "this cache needs more relax scratch than the library holds "
                                      "(kvc_relax_scratch_bytes > KVC_RELAX_NOALLOC_SCRATCH_BYTES)"
                                    : "relax scratch too small");
  const int32_t n = h->st.n_valid(), ns = h->st.ns, S = h->S;
  if (n % S != 0 || ns % S != 0) return fail(KVC_EINVAL, "relax scores need whole frames in the cache");
  if (tail_frames < 1) return fail(KVC_EINVAL, "tail_frames must be >= 1");
  const int32_t n_cand = n / S - ns / S - tail_frames;
  if (n_cand < 1) return fail(KVC_EINVAL, "no candidate frame between the sink and the tail");
  if (n_cand + tail_frames > kvc::kRelaxMaxFrames)
    return fail(KVC_EUNSUPPORTED, "relax scores take at most 64 frames (candidates + tail)");
  const int32_t CH = h->D * h->geo.esz / 16;
  if (256 % CH != 0) return fail(KVC_EUNSUPPORTED, "head_dim not supported by the frame sums");
  kvc::RelaxArgs a{};
  a.keys = key_regions(h);
  a.ns = ns;
  a.hs = h->st.hs;
  a.S_tok = std::max(1, h->st.S_tok);
  a.nw = h->st.nw;
  a.hw = h->st.hw;
  a.W_tok = h->st.W_tok;
  a.first = ns / S;
  a.n_cand = n_cand;
  a.n_tail = tail_frames;
  a.nsl = relax_slices(h);
  const size_t nfc = (size_t)(h->st.S_tok + h->st.W_tok) / S;
  a.part = (float*)scratch;
  a.xsum = (float*)((char*)scratch + align_up(nfc * a.nsl * h->H * h->D * 4));
  a.gram = (float*)((char*)a.xsum + align_up(nfc * h->H * h->D * 4));
  a.scores = scores;
  a.weight = weight;
  a.geo = h->geo;
  hipError_t e = hipSuccess;
  if (h->cflags & KVC_CREATE_RAW_KEYS)
    e = launch_placed_ka(h, (char*)a.gram + align_up((size_t)kvc::kRelaxMaxFrames * kvc::kRelaxMaxFrames * 4),
                         &a.keys);
  if (e == hipSuccess) e = kvc::launch_relax(a, h->stream);
  return device_result(h, e, "relax scores");
}

kvc_status kvc_relax_scores(kvc_handle h, int32_t tail_frames, float weight, float* scores, void* scratch,
                            size_t scratch_bytes) {
  if (kvc_status s = check(h)) return s;
  if (!scratch) return fail(KVC_EINVAL, "null argument");
  if ((uintptr_t)scratch % kAlign != 0) return fail(KVC_EINVAL, "scratch must be 256-byte aligned");
  return relax_impl(h, tail_frames, weight, scores, scratch, scratch_bytes, false);
}

kvc_status kvc_relax_scores_noalloc(kvc_handle h, int32_t tail_frames, float weight, float* scores) {
  if (kvc_status s = check(h)) return s;
  if (kvc_relax_scratch_bytes(h) > kvc::kRelaxNoallocScratch)
    return fail(KVC_ENOMEM, "this cache needs more relax scratch than the library holds "
                            "(kvc_relax_scratch_bytes > KVC_RELAX_NOALLOC_SCRATCH_BYTES)");
  void* p = nullptr;
  const hipError_t e = kvc::relax_noalloc_scratch(&p);
  if (e != hipSuccess) return fail(KVC_EDEVICE, std::string("relax scratch address: ") + hipGetErrorString(e));
  return relax_impl(h, tail_frames, weight, scores, p, kvc::kRelaxNoallocScratch, true);
}

kvc_status kvc_set_attention_limit(kvc_handle h, int32_t max_keys) {
  if (kvc_status s = check(h)) return s;
  if (max_keys < 0) return fail(KVC_EINVAL, "max_keys must be >= 0");
  if (h->max_keys != max_keys) ++h->epoch;
  h->max_keys = max_keys;
  return KVC_OK;
}

kvc_status kvc_set_memory_rates(kvc_handle h, float alpha_long, float alpha_short) {
  if (kvc_status s = check(h)) return s;
  if (!(h->cflags & KVC_CREATE_MEMORY)) return fail(KVC_EUNSUPPORTED, "no memory tokens (KVC_CREATE_MEMORY)");
  if (!(alpha_long >= 0.f && alpha_long <= 1.f && alpha_short >= 0.f && alpha_short <= 1.f))
    return fail(KVC_EINVAL, "memory rates outside [0, 1]");
  h->mem_alpha[0] = alpha_long;
  h->mem_alpha[1] = alpha_short;
  return KVC_OK;
}

kvc_status kvc_export_memory(kvc_handle h, void* k, void* v, int32_t* n_folded) {
  if (kvc_status s = check(h)) return s;
  if (!(h->cflags & KVC_CREATE_MEMORY)) return fail(KVC_EUNSUPPORTED, "no memory tokens (KVC_CREATE_MEMORY)");
  if (!k || !v || !n_folded) return fail(KVC_EINVAL, "null argument");
  kvc::MemExportArgs m{};
  m.sink = h->sink;
  m.mem_lo = h->L.S_tok;
  m.k = k;
  m.v = v;
  m.geo = h->geo;
  hipError_t e = kvc::launch_mem_export(m, h->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
  if (kvc_status s = device_result(h, e, "export memory")) return s;
  *n_folded = h->mem_frames;
  return KVC_OK;
}

static kvc_status compact_layers(const kvc_handle* hs, int32_t nl, const int32_t* keep_idx, int32_t n_keep) {
  if (kvc_status s = check_layers(hs, nl)) return s;
  kvc_handle h = hs[0];
  if (h->cflags & KVC_CREATE_MEMORY) return fail(KVC_EUNSUPPORTED, "compact is not available with memory tokens");
  if (!(h->cflags & KVC_CREATE_COMPACT)) return fail(KVC_EUNSUPPORTED, "compact needs KVC_CREATE_COMPACT");
  kvc::RingState nx = h->st;
  std::vector<int32_t> src;
  std::string err;
  if (!kvc::plan_compact(nx, keep_idx, n_keep, &src, &err)) return fail(KVC_EINVAL, err);
  hipError_t e = hipSuccess;
  if (!src.empty()) {
    // The source slots go up once, into the first layer's workspace, and serve every layer: the host
    // writes them to one half of the pinned staging buffer and a small kernel copies them to the device
    // (a stream copy of a few tens of KB costs several times longer).  The half used two calls ago is
    // rewritten only after its staging kernel has run.
    const int half = h->keep_half;
    int32_t* stage = h->keep_pinned + (size_t)half * h->L.WP;
    if (h->keep_pending[half]) {
      e = hipEventSynchronize(h->keep_evt[half]);
      h->keep_pending[half] = false;
    }
    if (e == hipSuccess) {
      std::memcpy(stage, src.data(), src.size() * 4);
      e = kvc::launch_stage_idx(h->keep_pinned_dev + (size_t)half * h->L.WP, h->keep_dev, (int32_t)src.size(),
                                h->stream);
    }
    if (e == hipSuccess) {
      e = hipEventRecord(h->keep_evt[half], h->stream);
      h->keep_pending[half] = e == hipSuccess;
      h->keep_half = half ^ 1;
    }
    if (e == hipSuccess) {
      kvc::CompactArgs a{};
      a.layers = nl;
      a.layer_stride = h->layer_stride;
      a.src = h->win[h->st.win_buf];
      a.dst = h->win[h->st.win_buf ^ 1];
      a.idx = h->keep_dev;
      a.n = (int32_t)src.size();
      a.geo = h->geo;
      e = kvc::launch_compact(a, h->stream);
    }
  }
  if (kvc_status s = device_result_layers(hs, nl, e, "compact")) return s;
  for (int32_t i = 0; i < nl; ++i) {
    hs[i]->st = nx;
    ++hs[i]->epoch;
  }
  return KVC_OK;
}

kvc_status kvc_compact(kvc_handle h, const int32_t* keep_idx, int32_t n_keep) {
  return compact_layers(&h, 1, keep_idx, n_keep);
}

kvc_status kvc_compact_layers(const kvc_handle* layers, int32_t n_layers, const int32_t* keep_idx, int32_t n_keep) {
  return compact_layers(layers, n_layers, keep_idx, n_keep);
}

static kvc_status sink_push_layers(const kvc_handle* hs, int32_t nl, int32_t bank_frame, int32_t n_frames,
                                   int32_t t_index) {
  if (kvc_status s = check_layers(hs, nl)) return s;
  kvc_handle h = hs[0];
  if (h->cflags & KVC_CREATE_MEMORY) return fail(KVC_EUNSUPPORTED, "sink push is not available with memory tokens");
  if (h->L.bank_tok == 0) return fail(KVC_ESTATE, "no bank (bank_frames was 0)");
  if (h->st.global_end < h->L.bank_tok) return fail(KVC_ESTATE, "bank not complete yet");
  if (bank_frame < 0 || n_frames < 1 || (int64_t)(bank_frame + n_frames) * h->S > h->L.bank_tok)
    return fail(KVC_EINVAL, "bank frame range");
  const int32_t b0 = bank_frame * h->S;
  kvc::RingState nx = h->st;
  std::vector<kvc::Seg> segs;
  std::string err;
  if (!kvc::plan_sink_push(nx, n_frames, b0, t_index, &segs, &err))
    return fail(h->st.ns != h->st.S_tok || h->st.S_tok == 0 ? KVC_ESTATE : KVC_EINVAL, err);
  const int64_t D = h->D;
  const char* bk = (const char*)h->bank_k + (size_t)b0 * D * h->geo.esz;
  const char* bv = (const char*)h->bank_v + (size_t)b0 * D * h->geo.esz;
  const int64_t head = (int64_t)h->L.bank_tok * D;
  // the bank is in each layer's workspace: sources move with the layer too
  hipError_t e = launch_segments(h, segs, bk, bv, D, head, D, head, t_index, b0, 0, 0, nl, h->layer_stride,
                                 h->layer_stride);
  if (kvc_status s = device_result_layers(hs, nl, e, "sink_push")) return s;
  for (int32_t i = 0; i < nl; ++i) {
    hs[i]->st = nx;
    ++hs[i]->epoch;
  }
  return KVC_OK;
}

kvc_status kvc_sink_push(kvc_handle h, int32_t bank_frame, int32_t n_frames, int32_t t_index) {
  return sink_push_layers(&h, 1, bank_frame, n_frames, t_index);
}

kvc_status kvc_sink_push_layers(const kvc_handle* layers, int32_t n_layers, int32_t bank_frame, int32_t n_frames,
                                int32_t t_index) {
  return sink_push_layers(layers, n_layers, bank_frame, n_frames, t_index);
}

kvc_status kvc_info(kvc_handle h, kvc_info_t* out) {
  if (!h || !out) return fail(KVC_EINVAL, "null argument");
  const kvc::RingState& s = h->st;
  std::memset(out, 0, sizeof(*out));
  out->capacity = s.S_tok + s.W_tok;
  out->n_valid = s.n_valid();
  out->sink_tokens = s.S_tok;
  out->window_tokens = s.W_tok;
  out->sink_filled = s.ns;
  out->window_filled = s.nw;
  out->sink_head = s.hs;
  out->window_head = s.hw;
  out->global_end = s.global_end;
  out->newest_valid = s.newest_valid ? 1 : 0;
  out->newest_frames = s.newest_valid ? s.newest_frames : 0;
  if (s.newest_valid) {
    const kvc::Seg& s0 = s.newest_segs.front();
    out->newest_t = s.t_at(s0.region, s0.dst) - s0.src / h->S;
    out->newest_g = s.newest_g;
  }
  out->bank_tokens = h->L.bank_tok;
  out->bank_complete = (h->L.bank_tok > 0 && s.global_end >= h->L.bank_tok) ? 1 : 0;
  out->window_buffer = s.win_buf;
  return KVC_OK;
}

kvc_status kvc_slot_times(kvc_handle h, int32_t* t, int64_t* g) {
  if (!h) return fail(KVC_EINVAL, "null handle");
  h->st.logical_times(t, g);
  return KVC_OK;
}

kvc_status kvc_export(kvc_handle h, void* k, void* v, int32_t* t, int64_t* g) {
  if (kvc_status s = check(h)) return s;
  if (!k || !v || !t || !g) return fail(KVC_EINVAL, "null argument");
  kvc::ExportArgs a{};
  a.reg[0] = h->sink;
  a.reg[1] = cur_win(h);
  a.ns = h->st.ns;
  a.hs = h->st.hs;
  a.S_tok = std::max(1, h->st.S_tok);
  a.nw = h->st.nw;
  a.hw = h->st.hw;
  a.W_tok = h->st.W_tok;
  a.k = k;
  a.v = v;
  a.t = t;
  a.g = g;
  a.geo = h->geo;
  hipError_t e = kvc::launch_export(a, h->st.n_valid(), h->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
  return device_result(h, e, "export");
}

kvc_status kvc_export_tables(kvc_handle h, int32_t band, int32_t pos_lo, int32_t n_pos, float* out) {
  if (kvc_status s = check(h)) return s;
  if (!out || n_pos < 0) return fail(KVC_EINVAL, "bad argument");
  const int32_t Pt = h->L.dt / 2, Pb = h->L.bw / 2;
  const char* src;
  size_t row;
  if (band == 0) {
    if (pos_lo < -KVC_MAX_POS || pos_lo + n_pos - 1 > KVC_MAX_POS) return fail(KVC_EINVAL, "time positions");
    row = (size_t)Pt * 2 * 4;
    src = h->ws + h->L.tab_t + (size_t)(pos_lo + KVC_MAX_POS) * row;
  } else if (band == 1 || band == 2) {
    const int32_t lim = band == 1 ? h->grid_h : h->grid_w;
    if (pos_lo < 0 || pos_lo + n_pos > lim) return fail(KVC_EINVAL, "grid positions");
    row = (size_t)Pb * 2 * 4;
    src = h->ws + (band == 1 ? h->L.tab_h : h->L.tab_w) + (size_t)pos_lo * row;
  } else {
    return fail(KVC_EINVAL, "band must be 0, 1 or 2");
  }
  hipError_t e = hipStreamSynchronize(h->stream);
  if (e == hipSuccess) e = hipMemcpy(out, src, row * n_pos, hipMemcpyDeviceToHost);
  return device_result(h, e, "export_tables");
}

const char* kvc_last_error(void) { return g_err.c_str(); }

}  // extern "C"
