// kvc_kernels.hip -- HBM-bound kernels of libkvc for gfx950, and the general
// (non matrix-core) attention and scoring paths.
//
//   append_kernel   fused 3D RoPE of new keys + ring scatter of K and V
//                   (+ raw capture into the Rolling-Sink bank); also serves
//                   the Rolling-Sink push, whose source is the bank
//   retime_kernel   in-place time-band re-rotation by a per-slot delta
//   compact_kernel  gather of kept window entries into the other buffer
//   export_kernel   logical-order gather for inspection
//   attend_general  one thread per (query, head), any dtype / head_dim
//   score_*         per-entry attention mass, four small passes
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>

#include "kvc_common.hip.hpp"
#include "kvc_launch.hpp"

namespace kvc {

// ----------------------------------------------------------------------------
// zero fill
__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, size_t n16) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  for (; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint4*)p, n16);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// append.  One grid, two kinds of 256-thread blocks:
//   K blocks: 256/CH consecutive tokens of a segment x up to 20 heads; lanes
//     run over the row's 16-byte chunks first, so a wave reads whole 256-byte
//     source rows and writes consecutive destination rows of each head's key
//     planes; each thread keeps eight chunks (heads) in flight.
//   V blocks: one 64-slot tile x (256/(8*CH)) heads; thread (group of 8 slots,
//     chunk) loads eight tokens' chunk, transposes it in registers and writes
//     eight d-rows of the tile, so eight lanes fill one 128-byte tile row.
// All index arithmetic is 32-bit.
template <typename T>
__device__ __forceinline__ SegW pick_seg_k(const AppendArgs& a, int b) {
  SegW sg = a.seg[0];
#pragma unroll
  for (int i = 1; i < kMaxSegs; ++i)
    if (i < a.nseg && b >= a.seg[i].kb0) sg = a.seg[i];
  return sg;
}

template <typename T>
__device__ __forceinline__ SegW pick_seg_v(const AppendArgs& a, int b) {
  SegW sg = a.seg[0];
#pragma unroll
  for (int i = 1; i < kMaxSegs; ++i)
    if (i < a.nseg && b >= a.seg[i].vb0) sg = a.seg[i];
  return sg;
}

// Key blocks: KTB tokens x up to KHB heads.  Thread (token i, chunk c) owns
// chunk c of token i for every head of its block: the token's frame, grid
// position and the chunk's (cos, sin) pairs are computed once and reused for
// each head, and all KHB 16-byte loads are in flight before the first store
// (one round per thread: many blocks, no chain of dependent rounds).  KHB is
// 4, with non-temporal loads (measured at 40 heads: 4 with those loads beats 8
// with plain ones by 4 %, and 8 with them is slower still).
constexpr int kAppendKHB = 4;

template <typename T, int D>
struct AppendShape {
  static constexpr int E = Elem<T>::E;
  static constexpr int CH = D / E;          // 16-byte chunks per row
  static constexpr int KTB = 256 / CH;      // tokens per key block
  // value blocks: VT = 8 tokens per thread (one 16-byte store per dim for bf16; 4 tokens with 8-byte stores
  // measured 4-12 % slower), VG token groups per tile, HPB heads per block
  static constexpr int VT = 8;
  static constexpr int VG = kTile / VT;
  static constexpr int HPB = 256 / (VG * CH);
  static_assert(HPB >= 1, "a value block holds a head's tile");
};

template <typename T, int D, int KHB>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  using Sh = AppendShape<T, D>;
  constexpr int E = Sh::E, CH = Sh::CH, KTB = Sh::KTB, HPB = Sh::HPB, HU = KHB;
  const Geo& g = a.geo;
  const int tid = threadIdx.x;
  int b = blockIdx.x;
  if (blockIdx.y > 0) {
    const int64_t off = (int64_t)blockIdx.y * a.layer_stride, soff = (int64_t)blockIdx.y * a.src_stride;
    a.reg[0] = layer_region(a.reg[0], off);
    a.reg[1] = layer_region(a.reg[1], off);
    a.bank_k = (char*)a.bank_k + off;
    a.bank_v = (char*)a.bank_v + off;
    a.k = (const char*)a.k + soff;
    a.v = (const char*)a.v + soff;
  }
  if (b < a.nkb) {
    const SegW sg = pick_seg_k<T>(a, b);
    const RegionPtrs R = sg.region == 0 ? a.reg[0] : a.reg[1];
    const int local = b - sg.kb0;
    const int nhg = (g.H + KHB - 1) / KHB;
    const int hg = local % nhg;
    const int i = (local / nhg) * KTB + tid / CH;
    const int c = tid % CH;
    if (i >= sg.n) return;
    const int src = sg.src + i, slot = sg.dst + i;
    const int f = src / g.S, tok = src - f * g.S;
    const int t = a.t0 + f, hp = tok / g.grid_w, wp = tok - hp * g.grid_w;
    const int d0 = c * E;
    float cs[E / 2][2];
    bool rot[E / 2];
#pragma unroll
    for (int q = 0; q < E / 2; ++q) {
      pair_cs(g, a.tab, d0 + 2 * q, t, hp, wp, cs[q][0], cs[q][1]);
      rot[q] = !(a.time_raw && d0 + 2 * q < g.dt);     // raw-key cache: the time band stays raw
    }
    const bool bank = src >= a.bank_lo && src < a.bank_hi;
    const T* sp = (const T*)a.k + (int64_t)src * a.k_tok + d0;
    T* dp;
    int64_t dstride;
    if (d0 < g.DA) {
      dp = (T*)R.ka + (int64_t)slot * g.DA + d0;
      dstride = (int64_t)R.cap * g.DA;
    } else {
      dp = (T*)R.kb + (int64_t)slot * g.DB + (d0 - g.DA);
      dstride = (int64_t)R.cap * g.DB;
    }
    T* bp = (T*)a.bank_k + ((int64_t)a.g0 + src) * D + d0;
    const int64_t bstride = (int64_t)a.bank_tok * D;
    const int h_lo = hg * KHB, h_hi = min(g.H, h_lo + KHB);
    for (int h0 = h_lo; h0 < h_hi; h0 += HU) {
      Vec16<T> x[HU];
#pragma unroll
      for (int u = 0; u < HU; ++u)
        if (h0 + u < h_hi) ld16<KHB <= 4>(x[u], sp + (int64_t)(h0 + u) * a.k_head);
#pragma unroll
      for (int u = 0; u < HU; ++u) {
        const int h = h0 + u;
        if (h >= h_hi) break;
        if (bank) *reinterpret_cast<uint4*>(bp + h * bstride) = x[u].u;
        float xf[E];
#pragma unroll
        for (int e = 0; e < E; ++e) xf[e] = Elem<T>::ld(x[u].e[e]);
#pragma unroll
        for (int q = 0; q < E / 2; ++q)
          if (rot[q]) rot_pair(xf[2 * q], xf[2 * q + 1], cs[q][0], cs[q][1]);
#pragma unroll
        for (int e = 0; e < E; ++e) x[u].e[e] = Elem<T>::st(xf[e]);
        *reinterpret_cast<uint4*>(dp + h * dstride) = x[u].u;
      }
    }
    if (c == 0 && hg == 0) {
      R.t[slot] = t;
      R.g[slot] = a.g0 + src;
    }
    return;
  }
  b -= a.nkb;
  const SegW sg = pick_seg_v<T>(a, b);
  const RegionPtrs R = sg.region == 0 ? a.reg[0] : a.reg[1];
  const int local = b - sg.vb0;
  const int nhb = (g.H + HPB - 1) / HPB;
  const int hb = local % nhb;
  const int tile = local / nhb + sg.dst / kTile;
  constexpr int VT = Sh::VT, VG = Sh::VG;
  const int grp = tid % VG;
  const int c = (tid / VG) % CH;
  const int h = hb * HPB + tid / (VG * CH);
  if (h >= g.H) return;
  const int slot0 = tile * kTile + grp * VT;
  // all VT loads issued before any is used: a slot outside the segment reads the segment's nearest row
  // (a valid address) and is zeroed after, instead of a load under a branch that would wait on its own
  Vec16<T> rows[VT];
  bool full = true;
#pragma unroll
  for (int j = 0; j < VT; ++j) {
    const int src = sg.src + min(max(slot0 + j - sg.dst, 0), sg.n - 1);
    ld16<true>(rows[j], (const T*)a.v + (int64_t)src * a.v_tok + (int64_t)h * a.v_head + c * E);
  }
#pragma unroll
  for (int j = 0; j < VT; ++j) {
    const int slot = slot0 + j;
    const bool ok = slot >= sg.dst && slot < sg.dst + sg.n;
    full = full && ok;
    if (!ok) rows[j].u = make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < VT; ++j) {
    const int slot = slot0 + j;
    const int src = sg.src + (slot - sg.dst);
    if (slot >= sg.dst && slot < sg.dst + sg.n && src >= a.bank_lo && src < a.bank_hi)
      *reinterpret_cast<uint4*>((T*)a.bank_v + ((int64_t)h * a.bank_tok + (a.g0 + src)) * D + c * E) = rows[j].u;
  }
  // dim c*E + e of the VT tokens: VT consecutive keys of one V^T row (8 or 16 bytes for bf16, 16 or 32 for
  // fp32), aligned to their size
  T* vb = (T*)R.v + v_index(h, R.cap, D, slot0, 0);
  constexpr int SB = VT * (int)sizeof(T);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    T* dst = vb + (size_t)(c * E + e) * kTile;
    if (full) {
      union {
        uint2 w2[SB / 8];
        T v[VT];
      } o;
#pragma unroll
      for (int j = 0; j < VT; ++j) o.v[j] = rows[j].e[e];
      if constexpr (SB == 8) {
        *reinterpret_cast<uint2*>(dst) = o.w2[0];
      } else {
#pragma unroll
        for (int q = 0; q < SB / 16; ++q)
          reinterpret_cast<uint4*>(dst)[q] = make_uint4(o.w2[2 * q].x, o.w2[2 * q].y, o.w2[2 * q + 1].x, o.w2[2 * q + 1].y);
      }
    } else {
#pragma unroll
      for (int j = 0; j < VT; ++j) {
        const int slot = slot0 + j;
        if (slot >= sg.dst && slot < sg.dst + sg.n) dst[j] = rows[j].e[e];
      }
    }
  }
}

// Blocks of the append grid for one segment list (host and kernel agree on
// these counts through the same constants).
template <typename T, int D>
static void append_blocks(AppendArgs& a, int khb) {
  using Sh = AppendShape<T, D>;
  constexpr int KTB = Sh::KTB, HPB = Sh::HPB;
  const int nhg = (a.geo.H + khb - 1) / khb;
  int kb = 0, vb = 0;
  for (int i = 0; i < a.nseg; ++i) {
    SegW& s = a.seg[i];
    s.kb0 = kb;
    s.vb0 = vb;
    kb += ((s.n + KTB - 1) / KTB) * nhg;
    const int t0 = s.dst / kTile, t1 = (s.dst + s.n - 1) / kTile;
    vb += (t1 - t0 + 1) * ((a.geo.H + HPB - 1) / HPB);
  }
  a.nkb = kb;
  a.nvb = vb;
}

template <typename T, int D>
static hipError_t append_launch(AppendArgs a, hipStream_t s) {
  constexpr int khb = kAppendKHB;
  append_blocks<T, D>(a, khb);
  const int blocks = a.nkb + a.nvb;
  if (blocks == 0) return hipSuccess;
  const unsigned layers = a.layers > 1 ? (unsigned)a.layers : 1u;
  hipLaunchKernelGGL((append_kernel<T, D, khb>), dim3(blocks, layers), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.nseg == 0) return hipSuccess;
  if (a.geo.esz == 2) return a.geo.D == 128 ? append_launch<uint16_t, 128>(a, s) : append_launch<uint16_t, 64>(a, s);
  return a.geo.D == 128 ? append_launch<float, 128>(a, s) : append_launch<float, 64>(a, s);
}

// ----------------------------------------------------------------------------
// retime: a block owns SLOTS consecutive slots of one physical range for
// every head; it reads their times, rotates the time band of every head's key
// by the slot's actual change (t' - t) and finally writes t'.  Thread (hq, p)
// owns chunk p % CA of slot p / CA in heads hq, hq + HL, hq + 2 HL, ... (HL
// head lanes of SLOTS * CA threads): its (cos, sin) pairs depend
// only on the slot's change and the chunk, so they are read from the table once
// and reused for all its heads; for each head the lane's threads cover the
// block's contiguous KA rows as one run of 16-byte chunks.  With 8 slots a
// block and up to 8 heads per thread, every thread issues all its loads in one
// round (40 heads: 5 head lanes x 8), and the many small blocks keep enough
// loads in flight on every CU; a loop over rounds per thread (32 slots a
// block, 5 rounds of 8 heads) left the stream about a quarter slower.  The
// block has as many head lanes as it needs: at least four heads per thread
// (with 12 heads, 3 lanes x 4 heads rather than 4 x 3, which measured 7 %
// slower), at most 256 threads.  With fewer than 24 heads a block takes 32
// slots instead of 8, so that it still moves tens of kilobytes (12 heads: 8
// slots a block measured 6 % slower than 32).
template <typename T, int D, int SLOTS>
struct RetimeShape {
  static constexpr int E = Elem<T>::E;
  static constexpr int DT = D - 4 * (D / 6);            // time band width
  static constexpr int CA = (DT + E - 1) / E;           // chunks per KA row (time band, padded)
  static constexpr int LANES = SLOTS * CA;              // threads per head lane
  static constexpr int HLMAX = 256 / LANES;             // head lanes of a 256-thread block
  static_assert(HLMAX >= 1, "one head lane fits a block");
  // heads per thread and head lanes for H heads (the block is lanes(H) * LANES threads)
  static constexpr int heads_per_thread(int H) {
    const int n = (H + HLMAX - 1) / HLMAX;
    return n < 4 ? (H < 4 ? H : 4) : n;
  }
  static constexpr int lanes(int H) { return (H + heads_per_thread(H) - 1) / heads_per_thread(H); }
};

// one thread's heads h0, h0 + HL, ..., HU of them, all loads issued before any is used (a head past the
// last is clamped to it: a repeated load, never stored; HL is chosen so that this is rare)
template <typename T, int D, int SLOTS, int HU>
__device__ __forceinline__ void retime_heads(const RetimeArgs& a, const T* base, T* obase, int64_t hstride, int h0,
                                             int HL, int H, int c, const int32_t* tslot, int tfix, bool fixed,
                                             bool placed) {
  using Sh = RetimeShape<T, D, SLOTS>;
  constexpr int E = Sh::E, DT = Sh::DT;
  Vec16<T> x[HU];
#pragma unroll
  for (int u = 0; u < HU; ++u) ld16<HU <= 4>(x[u], base + min(h0 + u * HL, H - 1) * hstride);
  // this chunk's rotation, shared by every head: the table row of the common change (the shift itself) is
  // fetched with the keys, and replaced only where a clamp or a placement makes the slot's change another
  // (every load unconditional: a pad pair past the band reads the band's last pair and is not used)
  auto rotation = [&](int dl, float (&cs)[E / 2][2]) {
    const float* tp = a.tab.tcs + ((size_t)(dl + a.tab.maxpos) * (DT / 2)) * 2;
#pragma unroll
    for (int q = 0; q < E / 2; ++q) {
      const int d = c * E + 2 * q;
      const float2 v = *reinterpret_cast<const float2*>(tp + min(d, DT - 2));
      cs[q][0] = d < DT ? v.x : 1.f;
      cs[q][1] = d < DT ? v.y : 0.f;
    }
  };
  float cs[E / 2][2];
  rotation(placed ? 0 : a.delta, cs);
  asm volatile("" ::: "memory");     // the slot's time is read after the key and table loads are issued
  const int t = fixed ? tfix : *tslot;
  const int tn = a.clamp0 ? max(0, t + a.delta) : t + a.delta;
  const int dl = placed ? t : tn - t;
  if (placed || dl != a.delta) rotation(dl, cs);
#pragma unroll
  for (int u = 0; u < HU; ++u) {
    float xf[E];
#pragma unroll
    for (int e = 0; e < E; ++e) xf[e] = Elem<T>::ld(x[u].e[e]);
#pragma unroll
    for (int q = 0; q < E / 2; ++q)
      if (c * E + 2 * q < DT) rot_pair(xf[2 * q], xf[2 * q + 1], cs[q][0], cs[q][1]);
#pragma unroll
    for (int e = 0; e < E; ++e) x[u].e[e] = Elem<T>::st(xf[e]);
  }
#pragma unroll
  for (int u = 0; u < HU; ++u)
    if (h0 + u * HL < H) *reinterpret_cast<uint4*>(obase + (h0 + u * HL) * hstride) = x[u].u;
}

template <typename T, int D, int SLOTS>
__global__ __launch_bounds__(256) void retime_kernel(RetimeArgs a) {
  using Sh = RetimeShape<T, D, SLOTS>;
  constexpr int E = Sh::E, CA = Sh::CA, LANES = Sh::LANES;
  const Geo& g = a.geo;
  const int b = blockIdx.x;
  RangeW rg = a.rng[0];
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (i < a.nrng && b >= a.rng[i].blk0) rg = a.rng[i];
  const int s0 = rg.lo + (b - rg.blk0) * SLOTS;
  const int ns = min(SLOTS, rg.lo + rg.n - s0);
  const RegionPtrs R = layer_region(rg.region == 0 ? a.reg[0] : a.reg[1], (int64_t)blockIdx.y * a.layer_stride);
  const int tid = threadIdx.x;
  const bool placed = a.out_ka[0] != nullptr;      // out of place, by each slot's absolute time
  const int hq = tid / LANES, p = tid - (tid / LANES) * LANES;
  const int j = p / CA, c = p - (p / CA) * CA;
  if (j < ns && a.keys) {
    const T* base = (const T*)R.ka + ((int64_t)s0 + j) * (CA * E) + c * E;
    T* obase = placed ? (T*)a.out_ka[rg.region] + ((int64_t)s0 + j) * (CA * E) + c * E : (T*)base;
    const int64_t hstride = (int64_t)R.cap * (CA * E);
    // the slot's own time is read by each of its threads (no barrier before the key loads)
    const int32_t* ts = R.t + s0 + j;
    const bool fx = placed && rg.fixed;
    // heads per thread nh and head lanes hl, as the launch sized the block (block-uniform)
    const int nh = Sh::heads_per_thread(g.H), hl = Sh::lanes(g.H);
    if (hq < hl) {
      if (nh <= 1)
        retime_heads<T, D, SLOTS, 1>(a, base, obase, hstride, hq, hl, g.H, c, ts, rg.tfix, fx, placed);
      else if (nh <= 2)
        retime_heads<T, D, SLOTS, 2>(a, base, obase, hstride, hq, hl, g.H, c, ts, rg.tfix, fx, placed);
      else if (nh <= 3)
        retime_heads<T, D, SLOTS, 3>(a, base, obase, hstride, hq, hl, g.H, c, ts, rg.tfix, fx, placed);
      else if (nh <= 4)
        retime_heads<T, D, SLOTS, 4>(a, base, obase, hstride, hq, hl, g.H, c, ts, rg.tfix, fx, placed);
      else {     // rounds of 8 heads, then the rest (4 or fewer in a round of 4)
        int h0 = hq;
        for (; h0 + hl * 7 < g.H; h0 += hl * 8)
          retime_heads<T, D, SLOTS, 8>(a, base, obase, hstride, h0, hl, g.H, c, ts, rg.tfix, fx, placed);
        const int rest = h0 < g.H ? (g.H - h0 + hl - 1) / hl : 0;
        if (rest > 4)
          retime_heads<T, D, SLOTS, 8>(a, base, obase, hstride, h0, hl, g.H, c, ts, rg.tfix, fx, placed);
        else if (rest > 0)
          retime_heads<T, D, SLOTS, 4>(a, base, obase, hstride, h0, hl, g.H, c, ts, rg.tfix, fx, placed);
      }
    }
  }
  if (placed) return;
  __syncthreads();     // every thread has read its slot's old time
  if (tid < ns) {
    const int t = R.t[s0 + tid];
    R.t[s0 + tid] = a.clamp0 ? max(0, t + a.delta) : t + a.delta;
  }
}

template <typename T, int D, int SLOTS>
static void retime_launch(const RetimeArgs& a, dim3 grid, hipStream_t s) {
  using Sh = RetimeShape<T, D, SLOTS>;
  // at least SLOTS threads (they write the slots' times), at most 256
  const unsigned threads = (unsigned)max(SLOTS, Sh::lanes(a.geo.H) * Sh::LANES);
  hipLaunchKernelGGL((retime_kernel<T, D, SLOTS>), grid, dim3(threads), 0, s, a);
}

template <typename T, int D>
static void retime_launch(const RetimeArgs& a, dim3 grid, hipStream_t s) {
  constexpr int FEW = retime_slots(1, D, (int)sizeof(T));     // the slot count with few heads
  static_assert(FEW == 16 || FEW == 32, "slots per workgroup with few heads");
  if (retime_slots(a.geo.H, D, (int)sizeof(T)) == 8)
    retime_launch<T, D, 8>(a, grid, s);
  else
    retime_launch<T, D, FEW>(a, grid, s);
}

hipError_t launch_retime(const RetimeArgs& a, int32_t nblocks, hipStream_t s) {
  if (nblocks == 0) return hipSuccess;
  const dim3 grid(nblocks, a.layers > 1 ? (unsigned)a.layers : 1u);
  if (a.geo.esz == 2) {
    if (a.geo.D == 128)
      retime_launch<uint16_t, 128>(a, grid, s);
    else
      retime_launch<uint16_t, 64>(a, grid, s);
  } else {
    if (a.geo.D == 128)
      retime_launch<float, 128>(a, grid, s);
    else
      retime_launch<float, 64>(a, grid, s);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// compact: destination slot j <- source slot idx[j] (the two window buffers;
// idx unique, increasing except once where the kept logical entries cross the
// window ring's wrap).  Two block kinds in one launch:
//  * key blocks: KS destination slots x KHC heads; thread (slot, chunk) copies
//    that 16-byte chunk of the slot's key row for each of the block's heads
//    (all in flight) and, in the first head group, for chunk 0, the slot's t
//    and g;
//  * value blocks: 4 VR rows of one destination V^T tile (64 slots) of one
//    head.  A slot's value is a column of a source V^T tile (one element in
//    each 64-slot row), so lane l of every wave owns destination slot l of the
//    tile and each wave VR rows: the lanes of one load read the kept columns of
//    one source row (a few 128-byte lines, as the kept slots rise), and the
//    lanes of one store write a whole destination row.  All VR loads of a
//    thread are in flight before its stores.  Slots past n in the last tile
//    are written as zeros: attention reads whole tiles and weights those slots
//    by exactly 0, which needs finite values.
template <typename T, int D>
struct CompactShape {
  static constexpr int E = Elem<T>::E;
  static constexpr int CH = D / E;          // 16-byte chunks per key row
  static constexpr int KS = 256 / CH;       // destination slots per key block
  static constexpr int KHC = 2;             // heads per key block
  static constexpr int VR = 8;              // value rows per wave
  static constexpr int VP = D / (4 * VR);   // value blocks per destination tile and head
};

template <typename T, int D>
__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a) {
  using Sh = CompactShape<T, D>;
  constexpr int E = Sh::E, CH = Sh::CH, KS = Sh::KS, KHC = Sh::KHC, VR = Sh::VR, VP = Sh::VP;
  const Geo& g = a.geo;
  if (blockIdx.y > 0) {
    a.src = layer_region(a.src, (int64_t)blockIdx.y * a.layer_stride);
    a.dst = layer_region(a.dst, (int64_t)blockIdx.y * a.layer_stride);
  }
  const int tid = threadIdx.x;
  int b = blockIdx.x;
  if (b < a.nk) {
    const int nhg = (g.H + KHC - 1) / KHC;
    const int hg = b % nhg;
    const int j = (b / nhg) * KS + tid / CH;
    const int c = tid % CH;
    if (j >= a.n) return;
    const int sj = a.idx[j];
    if (c == 0 && hg == 0) {
      a.dst.t[j] = a.src.t[sj];
      a.dst.g[j] = a.src.g[sj];
    }
    const int d0 = c * E;
    const T* sp;
    T* dp;
    int64_t ss, ds;
    if (d0 < g.DA) {
      sp = (const T*)a.src.ka + (int64_t)sj * g.DA + d0;
      dp = (T*)a.dst.ka + (int64_t)j * g.DA + d0;
      ss = (int64_t)a.src.cap * g.DA;
      ds = (int64_t)a.dst.cap * g.DA;
    } else {
      sp = (const T*)a.src.kb + (int64_t)sj * g.DB + (d0 - g.DA);
      dp = (T*)a.dst.kb + (int64_t)j * g.DB + (d0 - g.DA);
      ss = (int64_t)a.src.cap * g.DB;
      ds = (int64_t)a.dst.cap * g.DB;
    }
    // native 16-byte vectors (HIP's uint4 class would land in private memory here)
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const int h0 = hg * KHC;
    v4u x[KHC];
#pragma unroll
    for (int u = 0; u < KHC; ++u)
      if (h0 + u < g.H) x[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(sp + (h0 + u) * ss));
#pragma unroll
    for (int u = 0; u < KHC; ++u)
      if (h0 + u < g.H) *reinterpret_cast<v4u*>(dp + (h0 + u) * ds) = x[u];
    return;
  }
  b -= (int)a.nk;
  const int NT = (a.n + kTile - 1) / kTile;
  const int vp = b % VP;
  b /= VP;
  const int h = b / NT, dt = b - (b / NT) * NT;
  constexpr int TE = D * kTile;                       // elements per V^T tile
  const int lane = tid & (kTile - 1), w = vp * 4 + tid / kTile;
  const int j = dt * kTile + lane;
  const bool ok = j < a.n;
  const int sj = ok ? a.idx[j] : 0;
  const T* sp = (const T*)a.src.v + ((size_t)h * (a.src.cap / kTile) + sj / kTile) * TE + (size_t)w * VR * kTile +
                sj % kTile;
  T* dp = (T*)a.dst.v + ((size_t)h * (a.dst.cap / kTile) + dt) * TE + (size_t)w * VR * kTile + lane;
  T x[VR];
#pragma unroll
  for (int r = 0; r < VR; ++r) x[r] = ok ? sp[r * kTile] : T(0);
#pragma unroll
  for (int r = 0; r < VR; ++r) dp[r * kTile] = x[r];
}

// Copy n int32 values from host-visible (pinned) memory to device memory: one
// read of each value over the bus, so the gather kernel then reads device memory.
__global__ __launch_bounds__(256) void stage_idx_kernel(const int32_t* __restrict__ src, int32_t* __restrict__ dst,
                                                        int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

hipError_t launch_stage_idx(const int32_t* host_visible, int32_t* dst, int32_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(stage_idx_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, host_visible, dst, n);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t compact_launch(CompactArgs a, hipStream_t s) {
  using Sh = CompactShape<T, D>;
  a.nk = (int64_t)((a.n + Sh::KS - 1) / Sh::KS) * ((a.geo.H + Sh::KHC - 1) / Sh::KHC);
  a.nv = (int64_t)a.geo.H * ((a.n + kTile - 1) / kTile) * Sh::VP;
  a.nt = 0;
  const int64_t blocks = a.nk + a.nv;
  if (blocks == 0) return hipSuccess;
  const unsigned layers = a.layers > 1 ? (unsigned)a.layers : 1u;
  hipLaunchKernelGGL((compact_kernel<T, D>), dim3((unsigned)blocks, layers), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  if (a.geo.esz == 2) return a.geo.D == 128 ? compact_launch<uint16_t, 128>(a, s) : compact_launch<uint16_t, 64>(a, s);
  return a.geo.D == 128 ? compact_launch<float, 128>(a, s) : compact_launch<float, 64>(a, s);
}

// ----------------------------------------------------------------------------
// export: logical entry l -> dense [l][h][D] K and V, t[l], g[l].
__device__ __forceinline__ void logical_slot(int l, int ns, int hs, int S_tok, int hw, int W_tok, int& region,
                                             int& slot) {
  if (l < ns) {
    region = 0;
    slot = (hs + l) % S_tok;
  } else {
    region = 1;
    slot = (hw + (l - ns)) % W_tok;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void export_kernel(ExportArgs a, int n) {
  constexpr int E = Elem<T>::E;
  const Geo& g = a.geo;
  const int CH = g.D / E;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)n * g.H * CH) return;
  const int c = (int)(gid % CH);
  const int64_t r = gid / CH;
  const int h = (int)(r % g.H);
  const int l = (int)(r / g.H);
  int region, slot;
  logical_slot(l, a.ns, a.hs, a.S_tok, a.hw, a.W_tok, region, slot);
  const RegionPtrs& R = a.reg[region];
  const int d0 = c * E;
  uint4 kk;
  if (d0 < g.DA)
    kk = *reinterpret_cast<const uint4*>((const T*)R.ka + ((int64_t)h * R.cap + slot) * g.DA + d0);
  else
    kk = *reinterpret_cast<const uint4*>((const T*)R.kb + ((int64_t)h * R.cap + slot) * g.DB + (d0 - g.DA));
  *reinterpret_cast<uint4*>((T*)a.k + ((int64_t)l * g.H + h) * g.D + d0) = kk;
  Vec16<T> vv;
#pragma unroll
  for (int e = 0; e < E; ++e) vv.e[e] = ((const T*)R.v)[v_index(h, R.cap, g.D, slot, d0 + e)];
  *reinterpret_cast<uint4*>((T*)a.v + ((int64_t)l * g.H + h) * g.D + d0) = vv.u;
  if (h == 0 && c == 0) {
    a.t[l] = R.t[slot];
    a.g[l] = R.g[slot];
  }
}

hipError_t launch_export(const ExportArgs& a, int32_t n_valid, hipStream_t s) {
  const int64_t total = (int64_t)n_valid * a.geo.H * (a.geo.D * a.geo.esz / 16);
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (a.geo.esz == 2)
    hipLaunchKernelGGL(export_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, a, n_valid);
  else
    hipLaunchKernelGGL(export_kernel<float>, dim3(blocks), dim3(256), 0, s, a, n_valid);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Query rotation shared by the general attention and the score passes:
// rotate row (token i, head h) of a raw [N][H][D] query tensor at the time of
// its frame and round it to the cache dtype.
template <typename T, int D>
__device__ __forceinline__ void load_rotated_query(const T* q, int i, int h, int t, const Geo& g, const Tables& tb,
                                                   float* out) {
  constexpr int E = Elem<T>::E;
  const int tok = i % g.S;
  const int hp = tok / g.grid_w, wp = tok % g.grid_w;
  const T* row = q + ((int64_t)i * g.H + h) * D;
#pragma unroll
  for (int c = 0; c < D / E; ++c) {
    Vec16<T> x;
    x.u = *reinterpret_cast<const uint4*>(row + c * E);
    float xf[E];
#pragma unroll
    for (int e = 0; e < E; ++e) xf[e] = Elem<T>::ld(x.e[e]);
    rotate_run<E>(xf, g, tb, c * E, t, hp, wp);
#pragma unroll
    for (int e = 0; e < E; ++e) out[c * E + e] = Elem<T>::ld(Elem<T>::st(xf[e]));
  }
}

// q . k_j for slot j of region r.  tr >= -maxpos: a raw-key cache, whose stored
// time band is first rotated to time tr and rounded, as the cache would store it.
template <typename T, int D>
__device__ __forceinline__ float key_dot(const float* qv, const KeyRegions& kr, int r, int h, int j, const Geo& g,
                                         const Tables& tb, int tr) {
  constexpr int E = Elem<T>::E;
  const T* ka = (const T*)kr.ka[r] + ((int64_t)h * kr.cap[r] + j) * g.DA;
  const T* kb = (const T*)kr.kb[r] + ((int64_t)h * kr.cap[r] + j) * g.DB;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D / E; ++c) {
    Vec16<T> x;
    const int d0 = c * E;
    x.u = d0 < g.DA ? *reinterpret_cast<const uint4*>(ka + d0) : *reinterpret_cast<const uint4*>(kb + (d0 - g.DA));
    float xf[E];
#pragma unroll
    for (int e = 0; e < E; ++e) xf[e] = Elem<T>::ld(x.e[e]);
    if (tr >= -tb.maxpos && d0 < g.dt) {
#pragma unroll
      for (int q = 0; q < E / 2; ++q) {
        const int d = d0 + 2 * q;
        if (d >= g.dt) break;
        const float* cs = tb.tcs + ((size_t)(tr + tb.maxpos) * (g.dt >> 1) + (d >> 1)) * 2;
        rot_pair(xf[2 * q], xf[2 * q + 1], cs[0], cs[1]);
        xf[2 * q] = Elem<T>::ld(Elem<T>::st(xf[2 * q]));
        xf[2 * q + 1] = Elem<T>::ld(Elem<T>::st(xf[2 * q + 1]));
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) acc = fmaf(qv[d0 + e], xf[e], acc);
  }
  return acc;
}

// General attention: one thread per (query row, head), online softmax.
template <typename T, int D>
__global__ __launch_bounds__(64) void attend_general_kernel(AttendArgs a) {
  const Geo& g = a.geo;
  const int64_t gid = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (gid >= (int64_t)a.Lq * g.H) return;
  const int h = (int)(gid % g.H);
  const int i = (int)(gid / g.H);
  float qv[D];
  load_rotated_query<T, D>((const T*)a.q, i, h, a.t0 + i / g.S, g, a.tab, qv);
  float m = -INFINITY, l = 0.f;
  float o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = 0.f;
  // block-causal: this row sees the first lim entries in logical order (sink region first)
  const int nall = a.keys.n[0] + a.keys.n[1];
  const int lim = a.causal_block > 0 ? min(nall, (i / a.causal_block + 1) * a.causal_block) : nall;
  for (int r = 0; r < 2; ++r) {
    const T* vbase = (const T*)a.keys.v[r];
    const int nr = min(a.keys.n[r], lim - (r == 0 ? 0 : a.keys.n[0]));
    for (int j = a.keys.lo[r]; j < nr; ++j) {
      int tr = INT32_MIN;
      if (a.raw) tr = (r == 0 && j >= a.mem_lo) ? a.mem_t[j - a.mem_lo >= g.S ? 1 : 0] : a.keys.t[r][j];
      const float s = key_dot<T, D>(qv, a.keys, r, h, j, g, a.tab, tr) * a.scale;
      const float mn = fmaxf(m, s);
      const float alpha = expf(m - mn);
      const float p = expf(s - mn);
      l = l * alpha + p;
      m = mn;
      const T* vrow = vbase + v_index(h, a.keys.cap[r], D, j, 0);
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = o[d] * alpha + p * Elem<T>::ld(vrow[(size_t)d * kTile]);
    }
  }
  T* out = (T*)a.out + ((int64_t)i * g.H + h) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) out[d] = Elem<T>::st(o[d] * inv);
  // the row's normaliser in log2 units of q.k: m is a maximum of the scaled scores (natural units)
  if (a.row_m != nullptr) a.row_m[(int64_t)h * a.Lq + i] = m * 1.4426950408889634f + log2f(l);
}

hipError_t launch_attend(const AttendArgs& a, uint32_t paths, hipStream_t s) {
  if (!(paths & kPathGeneral) && a.geo.esz == 2 && a.geo.D == 128) return launch_attend_mfma(a, paths, s);
  if (!(paths & kPathGeneral) && a.geo.esz == 2 && a.geo.D == 64 && !a.raw) return launch_attend_mfma64(a, s);
  const int64_t total = (int64_t)a.Lq * a.geo.H;
  const unsigned blocks = (unsigned)((total + 63) / 64);
  if (a.geo.esz == 2) {
    if (a.geo.D == 128)
      hipLaunchKernelGGL((attend_general_kernel<uint16_t, 128>), dim3(blocks), dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((attend_general_kernel<uint16_t, 64>), dim3(blocks), dim3(64), 0, s, a);
  } else {
    if (a.geo.D == 128)
      hipLaunchKernelGGL((attend_general_kernel<float, 128>), dim3(blocks), dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((attend_general_kernel<float, 64>), dim3(blocks), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// score: (1) rotate the query window, (2) per-row max and sum of exp, (3) per
// (key, head) column sum of the normalized probabilities, (4) sum over heads
// into logical order.
// rotated queries to scratch as [H][Nq][D] in fp32, for the general passes (the
// values are already rounded to the cache dtype)
template <typename T, int D>
__global__ __launch_bounds__(64) void score_rot_kernel(ScoreArgs a) {
  const Geo& g = a.geo;
  const int64_t gid = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (gid >= (int64_t)a.Nq * g.H) return;
  const int h = (int)(gid % g.H);
  const int i = (int)(gid / g.H);
  float qv[D];
  load_rotated_query<T, D>((const T*)a.q, i, h, a.qt[i / g.S], g, a.tab, qv);
  float* dst = a.qh + ((int64_t)h * a.Nq + i) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) dst[d] = qv[d];
}

// The matrix-core passes' rotation, to bf16 (exact: the values are already rounded): one thread per
// 16-byte chunk of a (row, head) query, so that the loads and stores of consecutive threads are
// consecutive 16-byte pieces of one row (a thread per row writing it element by element, 64 rows apart
// across a wave, took 57 us at the C3 window).
template <int D>
__global__ __launch_bounds__(256) void score_rot_bf16_kernel(ScoreArgs a) {
  constexpr int E = Elem<uint16_t>::E, CH = D / E;
  const Geo& g = a.geo;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)a.Nq * g.H * CH) return;
  const int c = (int)(gid % CH);
  const int64_t r = gid / CH;                 // destination row h * Nq + i
  const int i = (int)(r % a.Nq), h = (int)(r / a.Nq);
  const int tok = i % g.S;
  Vec16<uint16_t> x;
  x.u = *reinterpret_cast<const uint4*>((const uint16_t*)a.q + ((int64_t)i * g.H + h) * D + c * E);
  float xf[E];
#pragma unroll
  for (int e = 0; e < E; ++e) xf[e] = Elem<uint16_t>::ld(x.e[e]);
  rotate_run<E>(xf, g, a.tab, c * E, a.qt[i / g.S], tok / g.grid_w, tok % g.grid_w);
#pragma unroll
  for (int e = 0; e < E; ++e) x.e[e] = Elem<uint16_t>::st(xf[e]);
  *reinterpret_cast<uint4*>((uint16_t*)a.qh + r * D + c * E) = x.u;
}

template <typename T, int D>
__global__ __launch_bounds__(64) void score_rows_kernel(ScoreArgs a) {
  const Geo& g = a.geo;
  const int64_t gid = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (gid >= (int64_t)a.Nq * g.H) return;
  const int h = (int)(gid / a.Nq);
  const int i = (int)(gid % a.Nq);
  float qv[D];
  const float* src = a.qh + ((int64_t)h * a.Nq + i) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) qv[d] = src[d];
  float m = -INFINITY, l = 0.f;
  for (int r = 0; r < 2; ++r)
    for (int j = 0; j < a.keys.n[r]; ++j) {
      const float s = key_dot<T, D>(qv, a.keys, r, h, j, g, a.tab, INT32_MIN) * a.scale;
      const float mn = fmaxf(m, s);
      l = l * expf(m - mn) + expf(s - mn);
      m = mn;
    }
  a.m[(int64_t)h * a.Nq + i] = m;
  a.l[(int64_t)h * a.Nq + i] = l;
}

template <typename T, int D>
__global__ __launch_bounds__(64) void score_cols_kernel(ScoreArgs a) {
  const Geo& g = a.geo;
  const int ncap = a.keys.cap[0] + a.keys.cap[1];
  const int64_t gid = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (gid >= (int64_t)ncap * g.H) return;
  const int h = (int)(gid / ncap);
  const int p = (int)(gid % ncap);
  const int r = p < a.keys.cap[0] ? 0 : 1;
  const int j = r == 0 ? p : p - a.keys.cap[0];
  if (j >= a.keys.n[r]) return;
  constexpr int E = Elem<T>::E;
  float kv[D];
  const T* ka = (const T*)a.keys.ka[r] + ((int64_t)h * a.keys.cap[r] + j) * g.DA;
  const T* kb = (const T*)a.keys.kb[r] + ((int64_t)h * a.keys.cap[r] + j) * g.DB;
#pragma unroll
  for (int d = 0; d < D; ++d) kv[d] = Elem<T>::ld(d < g.DA ? ka[d] : kb[d - g.DA]);
  (void)E;
  double acc = 0.0;
  for (int i = 0; i < a.Nq; ++i) {
    const float* qv = a.qh + ((int64_t)h * a.Nq + i) * D;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(qv[d], kv[d], s);
    s *= a.scale;
    // rows_given: a.m is the attention's log2 normaliser of the row (no separate row sum)
    acc += a.rows_given ? (double)exp2f(fmaf(s, 1.4426950408889634f, -a.m[(int64_t)h * a.Nq + i]))
                        : (double)(expf(s - a.m[(int64_t)h * a.Nq + i]) / a.l[(int64_t)h * a.Nq + i]);
  }
  a.part[(int64_t)h * ncap + p] = (float)acc;
}

__global__ __launch_bounds__(256) void score_reduce_kernel(ScoreArgs a) {
  const int ncap = a.keys.cap[0] + a.keys.cap[1];
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= ncap) return;
  const int r = p < a.keys.cap[0] ? 0 : 1;
  const int j = r == 0 ? p : p - a.keys.cap[0];
  if (j >= a.keys.n[r]) return;
  float acc = 0.f;
  for (int h = 0; h < a.geo.H; ++h) acc += a.part[(int64_t)h * ncap + p];
  int l;
  if (r == 0)
    l = (j - a.hs + a.S_tok) % a.S_tok;
  else
    l = a.ns + (j - a.hw + a.W_tok) % a.W_tok;
  a.scores[l] = acc;
}

template <typename T, int D>
static void score_launch_all(const ScoreArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.Nq * a.geo.H;
  const unsigned b1 = (unsigned)((rows + 63) / 64);
  hipLaunchKernelGGL((score_rot_kernel<T, D>), dim3(b1), dim3(64), 0, s, a);
  if (!a.rows_given) hipLaunchKernelGGL((score_rows_kernel<T, D>), dim3(b1), dim3(64), 0, s, a);
  const int64_t cols = (int64_t)(a.keys.cap[0] + a.keys.cap[1]) * a.geo.H;
  hipLaunchKernelGGL((score_cols_kernel<T, D>), dim3((unsigned)((cols + 63) / 64)), dim3(64), 0, s, a);
  const int ncap = a.keys.cap[0] + a.keys.cap[1];
  hipLaunchKernelGGL(score_reduce_kernel, dim3((unsigned)((ncap + 255) / 256)), dim3(256), 0, s, a);
}

hipError_t launch_score(const ScoreArgs& a, uint32_t paths, hipStream_t s) {
  if (!(paths & kPathGeneral) && a.geo.esz == 2 && (a.geo.D == 128 || a.geo.D == 64)) {
    const int64_t rows = (int64_t)a.Nq * a.geo.H;
    const int ch = a.geo.D / 8;              // 16-byte chunks per query row
    if (a.geo.D == 128)
      hipLaunchKernelGGL(score_rot_bf16_kernel<128>, dim3((unsigned)((rows * ch + 255) / 256)), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(score_rot_bf16_kernel<64>, dim3((unsigned)((rows * ch + 255) / 256)), dim3(256), 0, s, a);
    const hipError_t e = a.geo.D == 128 ? launch_score_mfma(a, (const uint16_t*)a.qh, s)
                                        : launch_score_mfma64(a, (const uint16_t*)a.qh, s);
    if (e != hipSuccess) return e;
    const int ncap = a.keys.cap[0] + a.keys.cap[1];
    hipLaunchKernelGGL(score_reduce_kernel, dim3((unsigned)((ncap + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (a.geo.esz == 2) {
    if (a.geo.D == 128)
      score_launch_all<uint16_t, 128>(a, s);
    else
      score_launch_all<uint16_t, 64>(a, s);
  } else {
    if (a.geo.D == 128)
      score_launch_all<float, 128>(a, s);
    else
      score_launch_all<float, 64>(a, s);
  }
  return hipGetLastError();
}

}  // namespace kvc

namespace kvc {

// ----------------------------------------------------------------------------
// MemRoPE memory fold.  Key blocks: thread (head, grid position p, 16-byte
// chunk c of the key row) walks the evicted frames oldest first, reading the
// chunk of the token at position p (consecutive threads read consecutive
// chunks and rows), and keeps both memories' fp32 state for its E dims in
// registers.  Value blocks: thread (head, dim d, positions p .. p + VW - 1)
// does the same on the tile-transposed values, where VW consecutive positions
// are VW consecutive slots of one tile row: one 16-byte load per frame (when
// the frame size, the ring head and size and the memory slots are multiples
// of VW; otherwise one position per thread).  Each update is
// M = a*M + (1-a)*E with the products and the sum rounded separately; the
// state is written back and the memory slots get it rounded to the cache
// dtype.  The frames go kFoldBatch at a time: their loads (and the state's)
// are issued together, then folded oldest first; a batch's loads past the
// last frame repeat the last frame's (valid addresses) and are not used, so no
// load sits under a branch of its own.
constexpr int kFoldBatch = 4;
template <typename T>
__device__ __forceinline__ float ema(float m, float e, float a, float b) {
#pragma clang fp contract(off)
  const float x = a * m;
  const float y = b * e;
  return x + y;
}

template <typename T, int W>
struct ValRun {       // W consecutive elements of type T
  union {
    uint4 u[(W * sizeof(T) + 15) / 16];
    T e[W];
  };
};

// value blocks: W positions per thread (W = 1: any geometry; W = 16 / sizeof(T): aligned runs)
template <typename T, int D, int W>
__device__ __forceinline__ void mem_fold_values(const MemFoldArgs& a, int64_t id) {
  const Geo& g = a.geo;
  const float al[2] = {a.alpha[0], a.alpha[1]};
  const float be[2] = {1.f - a.alpha[0], 1.f - a.alpha[1]};
  const int np = g.S / W;
  const int p = (int)(id % np) * W;
  const int64_t hd = id / np;
  if (hd >= (int64_t)g.H * D) return;
  const int d = (int)(hd % D), h = (int)(hd / D);
  float st[2][W] = {};
  if (!a.init) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float* sp = a.state_v + (((int64_t)m * g.H + h) * D + d) * g.S + p;
#pragma unroll
      for (int w = 0; w < W; ++w) st[m][w] = sp[w];
    }
  }
  for (int f0 = 0; f0 < a.n_frames; f0 += kFoldBatch) {
    ValRun<T, W> x[kFoldBatch];
#pragma unroll
    for (int u = 0; u < kFoldBatch; ++u) {
      const int f = min(f0 + u, a.n_frames - 1);
      const int slot = (a.hw + f * g.S + p) % a.W_tok;
      const T* src = (const T*)a.win.v + v_index(h, a.win.cap, D, slot, d);
      if (W * sizeof(T) >= 16) {
#pragma unroll
        for (int q = 0; q < (int)(W * sizeof(T) / 16); ++q) x[u].u[q] = reinterpret_cast<const uint4*>(src)[q];
      } else {
        x[u].e[0] = src[0];
      }
    }
    // every loaded frame is folded and the result kept only for real frames (a branch here would let the
    // compiler sink each load into it, one wait per frame)
#pragma unroll
    for (int u = 0; u < kFoldBatch; ++u) {
      const bool real = f0 + u < a.n_frames, first = f0 + u == 0 && a.init;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int w = 0; w < W; ++w) {
          const float e = Elem<T>::ld(x[u].e[w]);
          const float nx = first ? e : ema<T>(st[m][w], e, al[m], be[m]);
          st[m][w] = real ? nx : st[m][w];
        }
    }
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    float* sp = a.state_v + (((int64_t)m * g.H + h) * D + d) * g.S + p;
    ValRun<T, W> y;
    if (W % 4 == 0) {
#pragma unroll
      for (int w = 0; w < W; w += 4)
        *reinterpret_cast<float4*>(sp + w) = make_float4(st[m][w], st[m][w + 1], st[m][w + 2], st[m][w + 3]);
    } else {
#pragma unroll
      for (int w = 0; w < W; ++w) sp[w] = st[m][w];
    }
#pragma unroll
    for (int w = 0; w < W; ++w) y.e[w] = Elem<T>::st(st[m][w]);
    T* dst = (T*)a.sink.v + v_index(h, a.sink.cap, D, a.mem_lo + m * g.S + p, d);
    if (W * sizeof(T) >= 16) {
#pragma unroll
      for (int q = 0; q < (int)(W * sizeof(T) / 16); ++q) reinterpret_cast<uint4*>(dst)[q] = y.u[q];
    } else {
      dst[0] = y.e[0];
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void mem_fold_kernel(MemFoldArgs a, int nkb, int vec) {
  constexpr int E = Elem<T>::E, CH = D / E;
  const Geo& g = a.geo;
  const float al[2] = {a.alpha[0], a.alpha[1]};
  const float be[2] = {1.f - a.alpha[0], 1.f - a.alpha[1]};
  if ((int)blockIdx.x < nkb) {
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int c = (int)(id % CH);
    const int64_t hp = id / CH;
    if (hp >= (int64_t)g.H * g.S) return;
    const int p = (int)(hp % g.S), h = (int)(hp / g.S);
    const int d0 = c * E;
    float st[2][E] = {};
    if (!a.init) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const float* sp = a.state_k + (((int64_t)m * g.H + h) * g.S + p) * D + d0;
#pragma unroll
        for (int e = 0; e < E; ++e) st[m][e] = sp[e];
      }
    }
    for (int f0 = 0; f0 < a.n_frames; f0 += kFoldBatch) {
      Vec16<T> x[kFoldBatch];
#pragma unroll
      for (int u = 0; u < kFoldBatch; ++u) {
        const int slot = (a.hw + min(f0 + u, a.n_frames - 1) * g.S + p) % a.W_tok;
        const T* src = d0 < g.DA ? (const T*)a.win.ka + ((int64_t)h * a.win.cap + slot) * g.DA + d0
                                 : (const T*)a.win.kb + ((int64_t)h * a.win.cap + slot) * g.DB + (d0 - g.DA);
        ld16<true>(x[u], src);
      }
#pragma unroll
      for (int u = 0; u < kFoldBatch; ++u) {
        const bool real = f0 + u < a.n_frames, first = f0 + u == 0 && a.init;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float v = Elem<T>::ld(x[u].e[e]);
            const float nx = first ? v : ema<T>(st[m][e], v, al[m], be[m]);
            st[m][e] = real ? nx : st[m][e];
          }
      }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float* sp = a.state_k + (((int64_t)m * g.H + h) * g.S + p) * D + d0;
      Vec16<T> y;
#pragma unroll
      for (int e = 0; e < E; e += 4)
        *reinterpret_cast<float4*>(sp + e) = make_float4(st[m][e], st[m][e + 1], st[m][e + 2], st[m][e + 3]);
#pragma unroll
      for (int e = 0; e < E; ++e) y.e[e] = Elem<T>::st(st[m][e]);
      const int slot = a.mem_lo + m * g.S + p;
      T* dst = d0 < g.DA ? (T*)a.sink.ka + ((int64_t)h * a.sink.cap + slot) * g.DA + d0
                         : (T*)a.sink.kb + ((int64_t)h * a.sink.cap + slot) * g.DB + (d0 - g.DA);
      *reinterpret_cast<uint4*>(dst) = y.u;
    }
    return;
  }
  const int64_t id = (int64_t)(blockIdx.x - nkb) * 256 + threadIdx.x;
  if (vec)
    mem_fold_values<T, D, (int)(16 / sizeof(T))>(a, id);
  else
    mem_fold_values<T, D, 1>(a, id);
}


template <typename T, int D>
__global__ __launch_bounds__(256) void mem_export_kernel(MemExportArgs a) {
  const Geo& g = a.geo;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)2 * g.S * g.H * D) return;
  const int d = (int)(id % D);
  const int64_t jh = id / D;
  const int h = (int)(jh % g.H), j = (int)(jh / g.H);
  const int slot = a.mem_lo + j;
  const T kv = d < g.DA ? ((const T*)a.sink.ka)[((int64_t)h * a.sink.cap + slot) * g.DA + d]
                        : ((const T*)a.sink.kb)[((int64_t)h * a.sink.cap + slot) * g.DB + (d - g.DA)];
  ((T*)a.k)[id] = kv;
  ((T*)a.v)[id] = ((const T*)a.sink.v)[v_index(h, a.sink.cap, D, slot, d)];
}

template <typename T, int D>
static hipError_t mem_fold_launch(const MemFoldArgs& a, hipStream_t s) {
  constexpr int CH = D / Elem<T>::E, VW = 16 / (int)sizeof(T);
  // runs of VW positions are VW consecutive, aligned slots of one tile row in the window and the memory
  const bool vec = a.geo.S % VW == 0 && a.hw % VW == 0 && a.W_tok % VW == 0 && a.mem_lo % VW == 0 &&
                   kTile % VW == 0;
  const int64_t nk = (int64_t)a.geo.H * a.geo.S * CH, nv = (int64_t)a.geo.H * D * a.geo.S / (vec ? VW : 1);
  const int nkb = (int)((nk + 255) / 256), nvb = (int)((nv + 255) / 256);
  hipLaunchKernelGGL((mem_fold_kernel<T, D>), dim3(nkb + nvb), dim3(256), 0, s, a, nkb, vec ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_mem_fold(const MemFoldArgs& a, hipStream_t s) {
  if (a.n_frames <= 0) return hipSuccess;
  if (a.geo.esz == 2) return a.geo.D == 128 ? mem_fold_launch<uint16_t, 128>(a, s) : mem_fold_launch<uint16_t, 64>(a, s);
  return a.geo.D == 128 ? mem_fold_launch<float, 128>(a, s) : mem_fold_launch<float, 64>(a, s);
}

hipError_t launch_mem_export(const MemExportArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)2 * a.geo.S * a.geo.H * a.geo.D;
  const unsigned b = (unsigned)((n + 255) / 256);
  if (a.geo.esz == 2) {
    if (a.geo.D == 128)
      hipLaunchKernelGGL((mem_export_kernel<uint16_t, 128>), dim3(b), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((mem_export_kernel<uint16_t, 64>), dim3(b), dim3(256), 0, s, a);
  } else {
    if (a.geo.D == 128)
      hipLaunchKernelGGL((mem_export_kernel<float, 128>), dim3(b), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((mem_export_kernel<float, 64>), dim3(b), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace kvc
