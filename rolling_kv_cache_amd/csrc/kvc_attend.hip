// kvc_attend.hip -- chunk attention over the bounded cache on gfx950 matrix cores.
//
// out[i] = sum_j softmax_j(q_hat_i . k_j / sqrt(128)) v_j over every valid
// cached entry, no mask (Causal-Forcing article, section 3; LingBot-World 2.0
// article, "how the window rolls when full": queries read the whole window,
// which already holds the new block).
//
// Design (bf16 inputs, fp32 accumulation, head_dim 128):
//  * workgroup = 4 waves x 32 query rows; key tiles of 64 slots, double
//    buffered in LDS (16 KB K + 16 KB V^T per buffer) with one barrier per tile;
//  * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16, so every lane owns one query
//    row: the row max needs one cross-half exchange, the row sum none;
//  * the key rows fed to the MFMA are permuted inside each 32-key block (bits
//    2 and 3 of the row index swapped), which makes the S^T accumulator
//    registers exactly the B operand of O^T = V^T . P^T: P goes from fp32
//    registers to packed bf16 and straight into the second MFMA, no shuffles;
//  * V^T comes from the cache already tile-transposed, so both LDS operand
//    reads are single 16-byte loads, XOR-swizzled to be bank-conflict free;
//  * online softmax in the log2 domain (exp2 with log2(e)/sqrt(D) folded into
//    one FMA); the running max only moves when a tile's max exceeds it by more
//    than 8 (log2 units), so the O rescale is skipped on almost every tile;
//  * queries are rotated (3D RoPE, fp32, no FMA) and rounded to bf16 in the
//    prologue, exactly as the cache rotates keys;
//  * workgroup -> (head, query block) mapping is XCD-aware: consecutive
//    blocks of the same head land on the same XCD so they share its L2.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kvc_common.hip.hpp"
#include "kvc_launch.hpp"

namespace kvc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// native vector type for 16-byte moves (HIP's uint4 is a class that blocks
// scalar replacement and lands in private memory)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;                       // queries per workgroup
constexpr int kBN = 64;                        // keys per tile
constexpr int kKCh = 16;                       // 16-byte chunks per K row
constexpr int kVCh = 8;                        // 16-byte chunks per V^T row
constexpr int kTileU4 = kBN * kKCh + 128 * kVCh;
constexpr int kDA = 48, kDB = 80;              // key plane widths for head_dim 128

__device__ __forceinline__ int perm_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
__device__ __forceinline__ int kswz(int row) { return (row & 3) | (((row >> 3) & 1) << 2); }

struct TileRegs {
  u32x4_t k[4];
  u32x4_t v[4];
};

__device__ __forceinline__ void tile_load(TileRegs& tr, const KeyRegions& kr, int h, int r, int base, int tid) {
  // select with conditionals: a dynamic index into the argument block would be
  // lowered to a private-memory copy
  const uint16_t* ka = (const uint16_t*)(r == 0 ? kr.ka[0] : kr.ka[1]);
  const uint16_t* kb = (const uint16_t*)(r == 0 ? kr.kb[0] : kr.kb[1]);
  const uint16_t* vv = (const uint16_t*)(r == 0 ? kr.v[0] : kr.v[1]);
  const int cap = r == 0 ? kr.cap[0] : kr.cap[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ci = tid + 256 * i;
    const int row = ci >> 4, c = ci & 15;
    const int64_t slot = (int64_t)h * cap + base + row;
    tr.k[i] = c < 6 ? *reinterpret_cast<const u32x4_t*>(ka + slot * kDA + c * 8)
                    : *reinterpret_cast<const u32x4_t*>(kb + slot * kDB + (c - 6) * 8);
  }
  const uint16_t* vt = vv + (((int64_t)h * (cap / kTile) + base / kTile) * 128) * kTile;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ci = tid + 256 * i;
    tr.v[i] = *reinterpret_cast<const u32x4_t*>(vt + (int64_t)ci * 8);
  }
}

__device__ __forceinline__ void tile_store(const TileRegs& tr, u32x4_t* lds, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ci = tid + 256 * i;
    const int row = ci >> 4, c = ci & 15;
    lds[row * kKCh + (c ^ kswz(row))] = tr.k[i];
  }
  u32x4_t* lv = lds + kBN * kKCh;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ci = tid + 256 * i;
    const int d = ci >> 3, c = ci & 7;
    lv[d * kVCh + (c ^ (d & 7))] = tr.v[i];
  }
}

__global__ __launch_bounds__(256, 2) void attend_mfma_kernel(AttendArgs a, int mblocks, int total, int per_xcd,
                                                             int ntile0, int ntiles) {
  __shared__ u32x4_t lds[2][kTileU4];
  const int wg = blockIdx.x;
  const int lin = (wg & 7) * per_xcd + (wg >> 3);
  if (lin >= total) return;
  const Geo& g = a.geo;
  const int h = lin / mblocks;
  const int mb = lin - h * mblocks;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int qrow = mb * kBM + wave * 32 + l32;
  const int qc = min(qrow, a.Lq - 1);

  // ---- prologue: rotate this lane's 64 query elements and keep them as B operands
  bf16x8_t qf[8];
  {
    const int tok = qc % g.S;
    const int t = a.t0 + qc / g.S, hp = tok / g.grid_w, wp = tok % g.grid_w;
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)qc * g.H + h) * 128;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qp + ks * 16 + hl * 8);
      const uint32_t xw[4] = {x[0], x[1], x[2], x[3]};
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(xw[e] << 16);
        f[2 * e + 1] = __uint_as_float(xw[e] & 0xFFFF0000u);
      }
      rotate_run<8>(f, g, a.tab, ks * 16 + hl * 8, t, hp, wp);
      u32x4_t y;
      y[0] = (uint32_t)f2bf_rne(f[0]) | ((uint32_t)f2bf_rne(f[1]) << 16);
      y[1] = (uint32_t)f2bf_rne(f[2]) | ((uint32_t)f2bf_rne(f[3]) << 16);
      y[2] = (uint32_t)f2bf_rne(f[4]) | ((uint32_t)f2bf_rne(f[5]) << 16);
      y[3] = (uint32_t)f2bf_rne(f[6]) | ((uint32_t)f2bf_rne(f[7]) << 16);
      qf[ks] = __builtin_bit_cast(bf16x8_t, y);
    }
  }

  f32x16_t o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  const float c2 = a.scale * 1.4426950408889634f;

  TileRegs tr;
  tile_load(tr, a.keys, h, 0, 0, tid);
  tile_store(tr, lds[0], tid);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const bool has_next = it + 1 < ntiles;
    if (has_next) {
      const int nx = it + 1;
      const int r = nx < ntile0 ? 0 : 1;
      tile_load(tr, a.keys, h, r, (r == 0 ? nx : nx - ntile0) * kBN, tid);
    }
    const u32x4_t* lk = lds[buf];
    const u32x4_t* lv = lds[buf] + kBN * kKCh;

    // ---- S^T = K . Q^T  (two 32-key blocks)
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
      const int row = kb * 32 + perm_row(l32);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, lk[row * kKCh + ((ks * 2 + hl) ^ (l32 & 7))]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks], s[kb], 0, 0, 0);
      }
    }

    // ---- ragged tail of a region: mask keys past its valid count
    {
      const int r = it < ntile0 ? 0 : 1;
      const int base = (r == 0 ? it : it - ntile0) * kBN;
      const int nv = (r == 0 ? a.keys.n[0] : a.keys.n[1]) - base;
      if (nv < kBN) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb * 32 + perm_row((i >> 2) * 8 + hl * 4 + (i & 3));
            if (key >= nv) s[kb][i] = -INFINITY;
          }
      }
    }

    // ---- online softmax (log2 domain)
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kb][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    mt *= c2;
    const bool upd = mt > m + 8.f;
    if (__ballot(upd) != 0) {
      const float mn = upd ? mt : m;
      const float alpha = upd ? exp2f(m - mn) : 1.f;
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[d][i] *= alpha;
    }
    bf16x8_t pb[2][2];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][hf * 8 + j], c2, -m));
          psum += p;
          pb[kb][hf][j] = (__bf16)p;
        }
    lsum += psum;

    // ---- O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = db * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, lv[d * kVCh + ((ks * 2 + hl) ^ (l32 & 7))]);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ks >> 1][ks & 1], o[db], 0, 0, 0);
      }
    }

    if (has_next) tile_store(tr, lds[buf ^ 1], tid);
    __syncthreads();
  }

  // ---- epilogue: combine the two halves' row sums, normalize, store bf16
  const float lt = lsum + __shfl_xor(lsum, 32);
  const float inv = 1.f / lt;
  if (qrow < a.Lq) {
    uint16_t* op = (uint16_t*)a.out + ((int64_t)qrow * g.H + h) * 128;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        union {
          uint2 u;
          __bf16 b[4];
        } w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w.b[e] = (__bf16)(o[db][gq * 4 + e] * inv);
        *reinterpret_cast<uint2*>(op + db * 32 + gq * 8 + hl * 4) = w.u;
      }
  }
}

hipError_t launch_attend_mfma(const AttendArgs& a, hipStream_t s) {
  const int mblocks = (a.Lq + kBM - 1) / kBM;
  const int total = mblocks * a.geo.H;
  const int per_xcd = (total + 7) / 8;
  const int ntile0 = (a.keys.n[0] + kBN - 1) / kBN;
  const int ntile1 = (a.keys.n[1] + kBN - 1) / kBN;
  if (total == 0 || ntile0 + ntile1 == 0) return hipSuccess;
  KeyRegions kr = a.keys;
  AttendArgs b = a;
  // a region with no valid keys contributes no tiles; keep region 0 non-empty
  if (ntile0 == 0) {
    b.keys.ka[0] = kr.ka[1];
    b.keys.kb[0] = kr.kb[1];
    b.keys.v[0] = kr.v[1];
    b.keys.cap[0] = kr.cap[1];
    b.keys.n[0] = kr.n[1];
    b.keys.n[1] = 0;
    hipLaunchKernelGGL(attend_mfma_kernel, dim3(8 * per_xcd), dim3(256), 0, s, b, mblocks, total, per_xcd, ntile1,
                       ntile1);
  } else {
    hipLaunchKernelGGL(attend_mfma_kernel, dim3(8 * per_xcd), dim3(256), 0, s, b, mblocks, total, per_xcd, ntile0,
                       ntile0 + ntile1);
  }
  return hipGetLastError();
}

}  // namespace kvc
