// kvc_relax.hip -- Relax Forcing frame scores (rCM length-extrapolation article,
// strategy 5): History frames ranked by cosine alignment of their keys with the
// Tail plus a complement bonus.
//
//   frame_sum_kernel     per (frame, head, 256-token slice): the sum of the
//                        slice's stored keys, fp32.  This is the only pass over
//                        HBM: every key of the candidates and the Tail is read
//                        once, as whole 16-byte chunks of contiguous key rows.
//   frame_reduce_kernel  the slices of each frame added (fixed order).
//   frame_gram_kernel    one workgroup per frame pair: <x_i, x_j>.
//   relax_score_kernel   one workgroup: cosines from the Gram matrix, then
//                        w * alignment + (1 - w) * complement.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "kvc_common.hip.hpp"
#include "kvc_launch.hpp"

// Scratch of kvc_relax_scores_noalloc: each GPU the library runs on holds its
// own copy for the life of the process.  Host code never passes this name to a
// kernel (on the host it is a stand-in, not a device address); it uses the
// address hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) unsigned char scratch[kvc::kRelaxNoallocScratch];

namespace kvc {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t relax_noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));     // with this device current: its own copy
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

typedef uint32_t u32x4_r __attribute__((ext_vector_type(4)));

// logical entry -> (region, slot): the sink ring first, then the window ring
__device__ __forceinline__ void relax_phys(const RelaxArgs& a, int l, int& r, int& slot) {
  if (l < a.ns) {
    r = 0;
    slot = (a.hs + l) % a.S_tok;
  } else {
    r = 1;
    slot = (a.hw + (l - a.ns)) % a.W_tok;
  }
}

// Block = one (frame, head, slice).  Thread (row, chunk): chunk c of the
// token's key row (the KA plane's chunks, then the KB plane's), tokens row,
// row + TPI, ...  Chunk c holds dims [c*E, c*E + E) since DA = CA*E.
template <int ESZ>
__global__ __launch_bounds__(256) void frame_sum_kernel(RelaxArgs a) {
  constexpr int E = 16 / ESZ;
  __shared__ float red[256 * E];
  const Geo& g = a.geo;
  int b = blockIdx.x;
  const int s = b % a.nsl;
  b /= a.nsl;
  const int h = b % g.H;
  const int f = b / g.H;
  const int CA = g.DA / E, CH = (g.DA + g.DB) / E;
  const int TPI = 256 / CH;
  const int c = threadIdx.x % CH, row = threadIdx.x / CH;
  const int tok1 = min(g.S, (s + 1) * kRelaxSlice);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  if (row < TPI) {
    const int64_t l0 = (int64_t)(a.first + f) * g.S;
    // kTrip tokens per trip, their loads issued together (a missing token adds zeros); more per trip
    // costs occupancy (16 per trip was a third slower)
    constexpr int kTrip = 4;
    // the regions' planes by plain selects (an index into the argument struct would be a memory load
    // ahead of every key load)
    const uint8_t* pl[2];
    int cap[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      pl[r] = c < CA ? (const uint8_t*)a.keys.ka[r] + (int64_t)c * E * ESZ
                     : (const uint8_t*)a.keys.kb[r] + (int64_t)(c - CA) * E * ESZ;
      cap[r] = a.keys.cap[r];
    }
    const int64_t rstride = (c < CA ? g.DA : g.DB) * (int64_t)ESZ;
    for (int tk = s * kRelaxSlice + row; tk < tok1; tk += kTrip * TPI) {
      u32x4_r w[kTrip];
      // every load issued before the first is used: a token past the slice reads the slice's last token
      // (a valid address) and adds zeros
#pragma unroll
      for (int u = 0; u < kTrip; ++u) {
        int r, slot;
        relax_phys(a, (int)(l0 + min(tk + u * TPI, tok1 - 1)), r, slot);
        const int64_t rowi = (int64_t)h * (r ? cap[1] : cap[0]) + slot;
        w[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_r*>((r ? pl[1] : pl[0]) + rowi * rstride));
      }
#pragma unroll
      for (int u = 0; u < kTrip; ++u)
        if (tk + u * TPI >= tok1) w[u] = u32x4_r{0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < kTrip; ++u) {
        if (ESZ == 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] += __uint_as_float(w[u][i] << 16);
            acc[2 * i + 1] += __uint_as_float(w[u][i] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int i = 0; i < E; ++i) acc[i] += __uint_as_float(w[u][i]);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[threadIdx.x * E + e] = acc[e];
  __syncthreads();
  const int D = g.D;
  for (int d = threadIdx.x; d < D; d += 256) {
    float sum = 0.f;
    for (int q = 0; q < TPI; ++q) sum += red[q * D + d];
    a.part[(((int64_t)f * a.nsl + s) * g.H + h) * D + d] = sum;
  }
}

// x[f][e] = sum over the frame's slices of part (fixed order), one thread per
// element: spreads the slice reduction over the chip.
__global__ __launch_bounds__(256) void frame_reduce_kernel(RelaxArgs a) {
  const int L = a.geo.H * a.geo.D;
  const int nb = (L + 255) / 256;
  const int f = blockIdx.x / nb, e = (blockIdx.x % nb) * 256 + threadIdx.x;
  if (e >= L) return;
  const float* p = a.part + (int64_t)f * a.nsl * L + e;
  float x = 0.f;
#pragma unroll 8
  for (int sl = 0; sl < a.nsl; ++sl) x += p[(int64_t)sl * L];
  a.xsum[(int64_t)f * L + e] = x;
}

__device__ __forceinline__ float block_sum_256(float v, float* sh) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  return sh[0] + sh[1] + sh[2] + sh[3];
}

// One workgroup per upper-triangle pair (i <= j): G[i][j] = <x_i, x_j>.
__global__ __launch_bounds__(256) void frame_gram_kernel(RelaxArgs a) {
  __shared__ float sh[4];
  const int nf = a.n_cand + a.n_tail;
  int i = 0, rem = blockIdx.x;
  while (rem >= nf - i) {
    rem -= nf - i;
    ++i;
  }
  const int j = i + rem;
  const int L = a.geo.H * a.geo.D;
  const float* xi = a.xsum + (int64_t)i * L;
  const float* xj = a.xsum + (int64_t)j * L;
  float acc = 0.f;
#pragma unroll 8
  for (int e = threadIdx.x; e < L; e += 256) acc += xi[e] * xj[e];
  const float tot = block_sum_256(acc, sh);
  if (threadIdx.x == 0) a.gram[i * nf + j] = tot;
}

// One workgroup: G (upper triangle) staged in LDS, then one thread per
// candidate forms its cosines.  The Tail vector is the sum of the Tail
// frames, so its products are sums of G entries.
__global__ __launch_bounds__(1024) void relax_score_kernel(RelaxArgs a) {
  __shared__ float G[kRelaxMaxFrames * kRelaxMaxFrames];
  const int nf = a.n_cand + a.n_tail;
  for (int idx = threadIdx.x; idx < nf * nf; idx += 1024) {
    const int i = idx / nf, j = idx - i * nf;
    if (i <= j) G[idx] = a.gram[idx];
  }
  __syncthreads();
  auto gg = [&](int i, int j) { return i <= j ? G[i * nf + j] : G[j * nf + i]; };
  float tn = 0.f;                          // |x_T|^2
  for (int t = a.n_cand; t < nf; ++t)
    for (int u = a.n_cand; u < nf; ++u) tn += gg(t, u);
  for (int i = threadIdx.x; i < a.n_cand; i += 1024) {
    const float gi = gg(i, i);
    float at = 0.f;
    for (int t = a.n_cand; t < nf; ++t) at += gg(i, t);
    const float align = (gi > 0.f && tn > 0.f) ? at / sqrtf(gi * tn) : 0.f;
    float cs = 0.f;
    for (int j = 0; j < a.n_cand; ++j) {
      if (j == i) continue;
      const float gj = gg(j, j);
      if (gi > 0.f && gj > 0.f) cs += gg(i, j) / sqrtf(gi * gj);
    }
    const float comp = a.n_cand > 1 ? 1.f - cs / (float)(a.n_cand - 1) : 1.f;
    a.scores[i] = a.weight * align + (1.f - a.weight) * comp;
  }
}

hipError_t launch_relax(const RelaxArgs& a, hipStream_t s) {
  const int nf = a.n_cand + a.n_tail;
  const unsigned b1 = (unsigned)((int64_t)nf * a.geo.H * a.nsl);
  if (a.geo.esz == 2)
    hipLaunchKernelGGL(frame_sum_kernel<2>, dim3(b1), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(frame_sum_kernel<4>, dim3(b1), dim3(256), 0, s, a);
  const int L = a.geo.H * a.geo.D;
  hipLaunchKernelGGL(frame_reduce_kernel, dim3((unsigned)(nf * ((L + 255) / 256))), dim3(256), 0, s, a);
  hipLaunchKernelGGL(frame_gram_kernel, dim3((unsigned)(nf * (nf + 1) / 2)), dim3(256), 0, s, a);
  hipLaunchKernelGGL(relax_score_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvc
