// kvc_attend.hip -- chunk attention over the bounded cache on gfx950 matrix cores.
//
// out[i] = sum_j softmax_j(q_hat_i . k_j / sqrt(128)) v_j over every valid
// cached entry, no mask (Causal-Forcing article, section 3; LingBot-World 2.0
// article, "how the window rolls when full": queries read the whole window,
// which already holds the new block).
//
// Design (bf16 inputs, fp32 accumulation, head_dim 128):
//  * workgroup = 4 waves x 32 query rows; key tiles of 64 slots staged in LDS
//    (16 KB K + 16 KB V^T), double buffered, one barrier per tile;
//  * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16, so every lane owns one query
//    row: the row max needs one exchange between the wave's halves
//    (v_permlane32_swap), the row sum none;
//  * the key rows fed to the MFMA are permuted inside each 32-key block (bits
//    2 and 3 of the row index swapped), which makes the S^T accumulator
//    registers exactly the B operand of O^T = V^T . P^T: P goes from fp32
//    registers to packed bf16 and straight into the second MFMA;
//  * V^T comes from the cache already tile-transposed, so both LDS operand
//    reads are single 16-byte loads.  The XOR swizzles make every group of 16
//    consecutive lanes touch 16 distinct 16-byte bank slots (and every group of
//    8 lanes 8 distinct slots), for reads and for the tile stores;
//  * online softmax in the log2 domain (exp2 with log2(e)/sqrt(D) folded into
//    one FMA); the running max only moves when a tile's max exceeds it by more
//    than 8 (log2 units), so the O rescale is skipped on almost every tile; the
//    row sum is accumulated from the packed bf16 P with v_dot2_f32_bf16, i.e.
//    from the same rounded probabilities the P.V product uses;
//  * queries are rotated (3D RoPE, fp32, no FMA) and rounded to bf16 in the
//    prologue, exactly as the cache rotates keys;
//  * workgroup -> (head, query block) mapping is XCD-aware: consecutive
//    blocks of the same head land on the same XCD so they share its L2.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <string>

#include "kvc_common.hip.hpp"
#include "kvc_launch.hpp"

namespace kvc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// native vector type for 16-byte moves (HIP's uint4 is a class that blocks
// scalar replacement and lands in private memory)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;                       // queries per workgroup
constexpr int kBN = 64;                        // keys per tile
constexpr int kKCh = 16;                       // 16-byte chunks per K row
constexpr int kVCh = 8;                        // 16-byte chunks per V^T row
constexpr int kDA = 48, kDB = 80;              // key plane widths for head_dim 128
constexpr int kVTile = 128 * kTile;            // elements of one V^T tile

// swap bits 2 and 3 of a row index inside a 32-row block
__device__ __forceinline__ int perm_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
// K tile: chunk c of row r is stored at chunk c ^ kswz(r)
__device__ __forceinline__ int kswz(int row) { return perm_row(row & 31) & 15; }
// V^T tile (128-byte rows): chunk c of row d is stored at chunk c ^ vswz(d)
__device__ __forceinline__ int vswz(int d) { return (d ^ (d >> 3)) & 7; }

// exchange with the lane 32 apart: {own, partner} in some order
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per-thread source pointers of the register-staged tile loads.  Thread tid
// always moves chunk column (tid & 15) of K rows (tid >> 4) + 16 i, and the
// 16-byte pieces tid + 256 i of the contiguous V^T tile.
struct TilePtrs {
  const uint16_t* k[2];   // region r, base slot 0, row (tid >> 4)
  const uint16_t* v[2];   // region r, tile 0, piece tid
  int kstride;            // elements per key row of this thread's plane
};

__device__ __forceinline__ TilePtrs tile_ptrs(const KeyRegions& kr, int h, int tid) {
  TilePtrs p;
  const int c = tid & 15;
  p.kstride = c < 6 ? kDA : kDB;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint16_t* plane = c < 6 ? (const uint16_t*)kr.ka[r] + c * 8 : (const uint16_t*)kr.kb[r] + (c - 6) * 8;
    p.k[r] = plane + ((int64_t)h * kr.cap[r] + (tid >> 4)) * p.kstride;
    p.v[r] = (const uint16_t*)kr.v[r] + (int64_t)h * (kr.cap[r] / kTile) * kVTile + tid * 8;
  }
  return p;
}

struct TileRegs {
  u32x4_t k[4];
  u32x4_t v[4];
};

__device__ __forceinline__ void tile_load(TileRegs& tr, const TilePtrs& p, int r, int base) {
  const uint16_t* kp = (r == 0 ? p.k[0] : p.k[1]) + base * p.kstride;
  const uint16_t* vp = (r == 0 ? p.v[0] : p.v[1]) + (base / kTile) * kVTile;
#pragma unroll
  for (int i = 0; i < 4; ++i) tr.k[i] = *reinterpret_cast<const u32x4_t*>(kp + 16 * i * p.kstride);
#pragma unroll
  for (int i = 0; i < 4; ++i) tr.v[i] = *reinterpret_cast<const u32x4_t*>(vp + 2048 * i);
}

__device__ __forceinline__ void tile_store(const TileRegs& tr, u32x4_t* lk, u32x4_t* lv, int tid) {
  const int c = tid & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (tid >> 4) + 16 * i;
    lk[row * kKCh + (c ^ kswz(row))] = tr.k[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ci = tid + 256 * i;
    const int d = ci >> 3, cv = ci & 7;
    lv[d * kVCh + (cv ^ vswz(d))] = tr.v[i];
  }
}

// Direct-to-LDS loads (global_load_lds_dwordx4): lane `lane` of wave `wave`
// fetches the chunk that belongs at LDS position blk*64 + lane.
__device__ __forceinline__ void dma_k(const KeyRegions& kr, int h, int rg, int base, u32x4_t* lk, int tid) {
  const uint16_t* ka = (const uint16_t*)(rg == 0 ? kr.ka[0] : kr.ka[1]);
  const uint16_t* kb = (const uint16_t*)(rg == 0 ? kr.kb[0] : kr.kb[1]);
  const int cap = rg == 0 ? kr.cap[0] : kr.cap[1];
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = i * 4 + wave;
    const int p = blk * 64 + lane;
    const int row = p >> 4, c = (p & 15) ^ kswz(row);
    const int64_t slot = (int64_t)h * cap + base + row;
    const uint16_t* src = c < 6 ? ka + slot * kDA + c * 8 : kb + slot * kDB + (c - 6) * 8;
    __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)(lk + blk * 64), 16,
                                     0, 0);
  }
}

__device__ __forceinline__ void dma_v(const KeyRegions& kr, int h, int rg, int base, u32x4_t* lv, int tid) {
  const uint16_t* vv = (const uint16_t*)(rg == 0 ? kr.v[0] : kr.v[1]);
  const int cap = rg == 0 ? kr.cap[0] : kr.cap[1];
  const uint16_t* vt = vv + ((int64_t)h * (cap / kTile) + base / kTile) * kVTile;
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = i * 4 + wave;
    const int p = blk * 64 + lane;
    const int d = p >> 3, c = (p & 7) ^ vswz(d);
    __builtin_amdgcn_global_load_lds((const void*)(vt + d * 64 + c * 8),
                                     (__attribute__((address_space(3))) void*)(lv + blk * 64), 16, 0, 0);
  }
}

// Rotate this lane's 64 query elements (row qc, halves hl) and pack them as the
// eight B operands of S^T = K . Q^T.
__device__ __forceinline__ void load_query(bf16x8_t* qf, const AttendArgs& a, int h, int qc, int hl) {
  const Geo& g = a.geo;
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

__device__ __forceinline__ void qk_tile(f32x16_t* s, const u32x4_t* lk, const bf16x8_t* qf, int l32, int hl) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
    const int row = kb * 32 + perm_row(l32);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, lk[row * kKCh + ((ks * 2 + hl) ^ (l32 & 15))]);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks], s[kb], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void mask_tile(f32x16_t* s, int nv, int hl) {
  if (nv >= kBN) return;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kb * 32 + perm_row((i >> 2) * 8 + hl * 4 + (i & 3));
      if (key >= nv) s[kb][i] = -INFINITY;
    }
}

// Online softmax of one tile in the log2 domain; returns P packed to bf16 as
// the four B operands of O^T += V^T . P^T.
__device__ __forceinline__ void softmax_tile(const f32x16_t* s, f32x16_t* o, float& m, float& lsum, float c2,
                                             bf16x8_t pb[2][2]) {
  float mt = s[0][0];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kb][i]);
  mt = xhalf_max(mt) * c2;
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
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[kb][hf][j] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][hf * 8 + j], c2, -m));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x2_t pr = {pb[kb][hf][2 * j], pb[kb][hf][2 * j + 1]};
        lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, one, lsum, false);
      }
    }
}

__device__ __forceinline__ void pv_tile(f32x16_t* o, const u32x4_t* lv, bf16x8_t pb[2][2], int l32, int hl) {
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int d = db * 32 + l32;
    const int sw = vswz(d);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, lv[d * kVCh + ((ks * 2 + hl) ^ sw)]);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ks >> 1][ks & 1], o[db], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void store_out(const AttendArgs& a, const f32x16_t* o, float lsum, int qrow, int h, int hl) {
  const float inv = 1.f / xhalf_sum(lsum);
  if (qrow >= a.Lq) return;
  uint16_t* op = (uint16_t*)a.out + ((int64_t)qrow * a.geo.H + h) * 128;
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

struct TileSeq {
  int ntile0, ntiles;
  int n0, n1;
  __device__ __forceinline__ int region(int it) const { return it < ntile0 ? 0 : 1; }
  __device__ __forceinline__ int base(int it) const { return (it < ntile0 ? it : it - ntile0) * kBN; }
  __device__ __forceinline__ int valid(int it) const { return (it < ntile0 ? n0 : n1) - base(it); }
};

// ---------------------------------------------------------------------------
// Main kernel: register-staged prefetch of tile t+1 while tile t is computed.
__global__ __launch_bounds__(256, 2) void attend_mfma_kernel(AttendArgs a, int mblocks, int total, int per_xcd,
                                                             int ntile0, int ntiles) {
  __shared__ u32x4_t lks[2][kBN * kKCh];
  __shared__ u32x4_t lvs[2][128 * kVCh];
  const int wg = blockIdx.x;
  const int lin = (wg & 7) * per_xcd + (wg >> 3);
  if (lin >= total) return;
  const int h = lin / mblocks;
  const int mb = lin - h * mblocks;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int qrow = mb * kBM + wave * 32 + l32;
  const TileSeq ts{ntile0, ntiles, a.keys.n[0], a.keys.n[1]};

  bf16x8_t qf[8];
  load_query(qf, a, h, min(qrow, a.Lq - 1), hl);

  f32x16_t o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  const float c2 = a.scale * 1.4426950408889634f;

  const TilePtrs tp = tile_ptrs(a.keys, h, tid);
  TileRegs tr;
  tile_load(tr, tp, 0, 0);
  tile_store(tr, lks[0], lvs[0], tid);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const bool has_next = it + 1 < ntiles;
    if (has_next) tile_load(tr, tp, ts.region(it + 1), ts.base(it + 1));
    f32x16_t s[2];
    qk_tile(s, lks[buf], qf, l32, hl);
    mask_tile(s, ts.valid(it), hl);
    bf16x8_t pb[2][2];
    softmax_tile(s, o, m, lsum, c2, pb);
    pv_tile(o, lvs[buf], pb, l32, hl);
    if (has_next) tile_store(tr, lks[buf ^ 1], lvs[buf ^ 1], tid);
    __syncthreads();
  }
  store_out(a, o, lsum, qrow, h, hl);
}

// ---------------------------------------------------------------------------
// Software-pipelined variant: while the softmax of tile t runs on the VALU,
// the matrix cores already compute S^T(t+1); then O^T += V^T(t) P^T(t).  K
// tiles run one tile ahead of V tiles, each double buffered (same 64 KB of
// LDS), filled with direct-to-LDS loads.
__global__ __launch_bounds__(256, 2) void attend_pipe_kernel(AttendArgs a, int mblocks, int total, int per_xcd,
                                                             int ntile0, int ntiles) {
  __shared__ u32x4_t lks[2][kBN * kKCh];
  __shared__ u32x4_t lvs[2][128 * kVCh];
  const int wg = blockIdx.x;
  const int lin = (wg & 7) * per_xcd + (wg >> 3);
  if (lin >= total) return;
  const int h = lin / mblocks;
  const int mb = lin - h * mblocks;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int qrow = mb * kBM + wave * 32 + l32;
  const TileSeq ts{ntile0, ntiles, a.keys.n[0], a.keys.n[1]};

  bf16x8_t qf[8];
  load_query(qf, a, h, min(qrow, a.Lq - 1), hl);

  f32x16_t o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  const float c2 = a.scale * 1.4426950408889634f;

  dma_k(a.keys, h, ts.region(0), ts.base(0), lks[0], tid);
  dma_v(a.keys, h, ts.region(0), ts.base(0), lvs[0], tid);
  if (ntiles > 1) dma_k(a.keys, h, ts.region(1), ts.base(1), lks[1], tid);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16_t sc[2];
  qk_tile(sc, lks[0], qf, l32, hl);
  mask_tile(sc, ts.valid(0), hl);

  for (int it = 0; it < ntiles; ++it) {
    const bool has1 = it + 1 < ntiles;
    const bool has2 = it + 2 < ntiles;
    if (has2) dma_k(a.keys, h, ts.region(it + 2), ts.base(it + 2), lks[it & 1], tid);
    if (has1) dma_v(a.keys, h, ts.region(it + 1), ts.base(it + 1), lvs[(it + 1) & 1], tid);
    f32x16_t sn[2];
    if (has1) qk_tile(sn, lks[(it + 1) & 1], qf, l32, hl);
    bf16x8_t pb[2][2];
    softmax_tile(sc, o, m, lsum, c2, pb);
    pv_tile(o, lvs[it & 1], pb, l32, hl);
    if (has1) mask_tile(sn, ts.valid(it + 1), hl);
    if (has1) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (has1) {
      sc[0] = sn[0];
      sc[1] = sn[1];
    }
  }
  store_out(a, o, lsum, qrow, h, hl);
}

template <bool PIPE>
static hipError_t attend_launch(const AttendArgs& a, hipStream_t s) {
  const int mblocks = (a.Lq + kBM - 1) / kBM;
  const int total = mblocks * a.geo.H;
  const int per_xcd = (total + 7) / 8;
  const int ntile0 = (a.keys.n[0] + kBN - 1) / kBN;
  const int ntile1 = (a.keys.n[1] + kBN - 1) / kBN;
  if (total == 0 || ntile0 + ntile1 == 0) return hipSuccess;
  AttendArgs b = a;
  int n0 = ntile0, nt = ntile0 + ntile1;
  // a region with no valid keys contributes no tiles; keep region 0 non-empty
  if (ntile0 == 0) {
    b.keys.ka[0] = a.keys.ka[1];
    b.keys.kb[0] = a.keys.kb[1];
    b.keys.v[0] = a.keys.v[1];
    b.keys.cap[0] = a.keys.cap[1];
    b.keys.n[0] = a.keys.n[1];
    b.keys.n[1] = 0;
    n0 = ntile1;
    nt = ntile1;
  }
  if (PIPE)
    hipLaunchKernelGGL(attend_pipe_kernel, dim3(8 * per_xcd), dim3(256), 0, s, b, mblocks, total, per_xcd, n0, nt);
  else
    hipLaunchKernelGGL(attend_mfma_kernel, dim3(8 * per_xcd), dim3(256), 0, s, b, mblocks, total, per_xcd, n0, nt);
  return hipGetLastError();
}

hipError_t launch_attend_mfma(const AttendArgs& a, hipStream_t s) {
  const char* v = std::getenv("KVC_ATTEND_VARIANT");
  if (v && std::string(v) == "p") return attend_launch<true>(a, s);
  return attend_launch<false>(a, s);
}

}  // namespace kvc
