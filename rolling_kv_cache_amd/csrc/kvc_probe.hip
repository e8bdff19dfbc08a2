// kvc_probe.hip -- measurement probes for the benchmark (libkvc_probe.so, not
// part of libkvc): the sustained bf16 matrix-core rate with the shader clock
// it runs at, and the HBM read / copy / write ceilings of plain streaming
// kernels.  They give the board's own ceilings beside the published peaks.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Each wave runs `iters` rounds of four independent v_mfma_f32_32x32x16_bf16
// chains (operands held in registers).  Thread 0 of each block records the
// shader-clock and the constant-rate wall-clock ticks the block took.
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* out, int64_t* ticks) {
  const int tid = threadIdx.x;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((tid + i) & 7));
    b[i] = (__bf16)(0.002f * (float)((tid * 3 + i) & 7));
  }
  f32x16_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  const int64_t c0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  out[(size_t)blockIdx.x * 256 + tid] = s;
  __syncthreads();
  if (tid == 0) {
    ticks[blockIdx.x * 2] = clock64() - c0;
    ticks[blockIdx.x * 2 + 1] = wall_clock64() - w0;
  }
}

// Streaming kernels over n16 16-byte elements, grid-stride, four elements in
// flight per thread.  MODE 0: read (xor-reduce into a per-thread value),
// 1: copy, 2: write, 3: copy with non-temporal stores, 4: copy with
// non-temporal loads and stores.
template <int MODE>
__global__ __launch_bounds__(256) void hbm_probe_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                        size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  const u32x4_t fill = {1u, 2u, 3u, (uint32_t)threadIdx.x};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    u32x4_t x[4];
    if (MODE == 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = __builtin_nontemporal_load(&src[i + u * stride]);
    } else if (MODE != 2) {
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = src[i + u * stride];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (MODE == 0) acc ^= x[u];
      if (MODE == 1) dst[i + u * stride] = x[u];
      if (MODE == 2) dst[i + u * stride] = fill;
      if (MODE == 3 || MODE == 4) __builtin_nontemporal_store(x[u], &dst[i + u * stride]);
    }
  }
  for (; i < n16; i += stride) {
    if (MODE == 0) acc ^= src[i];
    if (MODE == 1) dst[i] = src[i];
    if (MODE == 2) dst[i] = fill;
    if (MODE == 3) __builtin_nontemporal_store(src[i], &dst[i]);
    if (MODE == 4) __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
  }
  if (MODE == 0) sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// One 16-byte element per thread, no loop (a grid of n16 / 256 workgroups):
// copy (MODE 5) or copy with non-temporal loads and stores (MODE 6).
template <int MODE>
__global__ __launch_bounds__(256) void hbm_flat_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                       size_t n16) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  if (MODE == 5) dst[i] = src[i];
  if (MODE == 6) __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
}

// One 16-byte element per thread, read and written back in place (MODE 7).
__global__ __launch_bounds__(256) void hbm_inplace_kernel(u32x4_t* __restrict__ p, size_t n16) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  u32x4_t x = p[i];
  x[0] += 1u;
  p[i] = x;
}

}  // namespace

extern "C" {

// MFMA probe: `blocks` workgroups of 4 waves, `iters` rounds of 4 MFMAs per
// wave.  out: device float[blocks * 256]; ticks: device int64[blocks * 2]
// (shader clocks, wall-clock ticks per block).  Returns a hipError_t code.
int kvc_probe_mfma(int blocks, int iters, float* out, int64_t* ticks, void* stream) {
  if (blocks < 1 || iters < 1 || !out || !ticks) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out, ticks);
  return (int)hipGetLastError();
}

// Wall-clock tick rate of the device (kHz), for the MFMA probe's clock figure.
int kvc_probe_wall_clock_khz(int device, int* khz) {
  return (int)hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, device);
}

// HBM probe over `bytes` (a multiple of 16): mode 0 read src, 1 copy src ->
// dst, 2 write dst, 3 copy with non-temporal stores, 4 copy with non-temporal
// loads and stores (modes 0-4: `blocks` workgroups of 256 threads,
// grid-stride), 5 copy and 6 copy with non-temporal loads and stores with one
// 16-byte element per thread, 7 read-modify-write of dst in place with one
// element per thread (`blocks` ignored); sink: device uint32[blocks * 256]
// (mode 0).
int kvc_probe_hbm(int mode, const void* src, void* dst, size_t bytes, int blocks, uint32_t* sink, void* stream) {
  if (blocks < 1 || bytes % 16 != 0 || mode < 0 || mode > 7) return (int)hipErrorInvalidValue;
  if ((mode != 2 && mode != 7 && !src) || (mode != 0 && !dst) || (mode == 0 && !sink)) return (int)hipErrorInvalidValue;
  const size_t n16 = bytes / 16;
  const hipStream_t s = (hipStream_t)stream;
  const u32x4_t* sp = (const u32x4_t*)src;
  u32x4_t* dp = (u32x4_t*)dst;
  switch (mode) {
    case 0: hipLaunchKernelGGL(hbm_probe_kernel<0>, dim3(blocks), dim3(256), 0, s, sp, dp, n16, sink); break;
    case 1: hipLaunchKernelGGL(hbm_probe_kernel<1>, dim3(blocks), dim3(256), 0, s, sp, dp, n16, sink); break;
    case 2: hipLaunchKernelGGL(hbm_probe_kernel<2>, dim3(blocks), dim3(256), 0, s, sp, dp, n16, sink); break;
    case 3: hipLaunchKernelGGL(hbm_probe_kernel<3>, dim3(blocks), dim3(256), 0, s, sp, dp, n16, sink); break;
    case 4: hipLaunchKernelGGL(hbm_probe_kernel<4>, dim3(blocks), dim3(256), 0, s, sp, dp, n16, sink); break;
    default: {
      const size_t nb = (n16 + 255) / 256;
      if (nb > 0x7FFFFFFFu) return (int)hipErrorInvalidValue;
      if (mode == 5)
        hipLaunchKernelGGL(hbm_flat_kernel<5>, dim3((unsigned)nb), dim3(256), 0, s, sp, dp, n16);
      else if (mode == 6)
        hipLaunchKernelGGL(hbm_flat_kernel<6>, dim3((unsigned)nb), dim3(256), 0, s, sp, dp, n16);
      else
        hipLaunchKernelGGL(hbm_inplace_kernel, dim3((unsigned)nb), dim3(256), 0, s, dp, n16);
      break;
    }
  }
  return (int)hipGetLastError();
}

}  // extern "C"
