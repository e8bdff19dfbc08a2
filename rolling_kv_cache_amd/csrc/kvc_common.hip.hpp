// kvc_common.hip.hpp -- device helpers shared by the HIP kernels of libkvc.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kvc_device.hpp"

namespace kvc {

// bfloat16 <-> float.  Storage rounding is round-to-nearest-even written out
// on the bit pattern so the cache contents do not depend on a conversion
// instruction's denormal mode.  A NaN is stored as the quiet NaN 0x7FC0 with
// its sign (adding the rounding bias to a NaN pattern could carry into the
// exponent and turn it into an infinity or a zero).
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f2bf_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return (uint16_t)((u & 0x7FFFFFFFu) > 0x7F800000u ? ((u >> 16) & 0x8000u) | 0x7FC0u : r);
}

template <typename T>
struct Elem;

template <>
struct Elem<uint16_t> {
  static constexpr int E = 8;   // elements per 16 bytes
  __device__ __forceinline__ static float ld(uint16_t x) { return bf2f(x); }
  __device__ __forceinline__ static uint16_t st(float f) { return f2bf_rne(f); }
};

template <>
struct Elem<float> {
  static constexpr int E = 4;
  __device__ __forceinline__ static float ld(float x) { return x; }
  __device__ __forceinline__ static float st(float f) { return f; }
};


typedef uint32_t u32x4_stream __attribute__((ext_vector_type(4)));

template <typename T>
union Vec16 {
  uint4 u;
  u32x4_stream n;       // the same 16 bytes as a native vector, for the non-temporal builtin
  T e[16 / sizeof(T)];
};

// 16-byte load into v, with the non-temporal hint when STREAM, for data a kernel streams through once.
// Measured on MI355X (a ~100 MB copy, MALL flushed): with one to four 16-byte loads in flight per thread
// the hint makes the copy about a third faster, with eight it makes it slower, and on the stores it makes
// no difference.  Each kernel uses it where its own measurement favoured it: the append (key blocks of
// four heads and value blocks of eight tokens: 42.2 -> 37.8 us at 40 heads) and the memory fold take
// it; the retime takes it only where a thread holds four or fewer rows.
template <bool STREAM, typename V>
__device__ __forceinline__ void ld16(V& v, const void* p) {
  if constexpr (STREAM)
    v.n = __builtin_nontemporal_load(reinterpret_cast<const u32x4_stream*>(p));
  else
    v.u = *reinterpret_cast<const uint4*>(p);
}

// One RoPE pair rotation with every product and sum rounded to fp32 (no fused
// multiply-add):  x' = (x*c) - (y*s),  y' = (x*s) + (y*c).
__device__ __forceinline__ void rot_pair(float& x, float& y, float c, float s) {
#pragma clang fp contract(off)
  const float xc = x * c;
  const float ys = y * s;
  const float xs = x * s;
  const float yc = y * c;
  x = xc - ys;
  y = xs + yc;
}

// (cos, sin) of the pair that starts at head dim d (even), for a token at
// time t and grid position (hp, wp).  Bands: [0, dt) time, [dt, dt+bw)
// height, [dt+bw, D) width; pair index restarts at 0 in each band.
__device__ __forceinline__ void pair_cs(const Geo& g, const Tables& tb, int d, int t, int hp, int wp, float& c,
                                        float& s) {
  const float* p;
  if (d < g.dt)
    p = tb.tcs + ((size_t)(t + tb.maxpos) * (g.dt >> 1) + (d >> 1)) * 2;
  else if (d < g.dt + g.bw)
    p = tb.hcs + ((size_t)hp * (g.bw >> 1) + ((d - g.dt) >> 1)) * 2;
  else
    p = tb.wcs + ((size_t)wp * (g.bw >> 1) + ((d - g.dt - g.bw) >> 1)) * 2;
  c = p[0];
  s = p[1];
}

// Rotate E consecutive elements (E/2 pairs) starting at head dim d0.
template <int E>
__device__ __forceinline__ void rotate_run(float* x, const Geo& g, const Tables& tb, int d0, int t, int hp, int wp) {
#pragma unroll
  for (int p = 0; p < E / 2; ++p) {
    float c, s;
    pair_cs(g, tb, d0 + 2 * p, t, hp, wp, c, s);
    rot_pair(x[2 * p], x[2 * p + 1], c, s);
  }
}

// The same region in the workspace `off` bytes further on (layer batching).
__device__ __forceinline__ RegionPtrs layer_region(RegionPtrs r, int64_t off) {
  r.ka = (char*)r.ka + off;
  r.kb = (char*)r.kb + off;
  r.v = (char*)r.v + off;
  r.t = (int32_t*)((char*)r.t + off);
  r.g = (int64_t*)((char*)r.g + off);
  return r;
}

// Index of the V element (head h, slot j, dim d) in the tile-transposed layout.
__device__ __forceinline__ size_t v_index(int h, int cap, int D, int j, int d) {
  return (((size_t)h * (cap / kTile) + (j / kTile)) * D + d) * kTile + (j % kTile);
}

}  // namespace kvc
