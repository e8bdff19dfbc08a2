// kvc_attend.hip -- chunk attention over the bounded cache on gfx950 matrix cores.
//
// out[i] = sum_j softmax_j(q_hat_i . k_j / sqrt(D)) v_j over every valid
// cached entry, no mask (Causal-Forcing article, section 3; LingBot-World 2.0
// article, "how the window rolls when full": queries read the whole window,
// which already holds the new block).
//
// Design (bf16 inputs, fp32 accumulation, head_dim 128):
//  * workgroup = 8 waves x 32 query rows (one per CU, two waves per SIMD); key
//    tiles of 64 slots staged in LDS (K + V^T, 35 KB with row padding), double
//    buffered, one barrier per tile;
//  * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16, so every lane owns one query
//    row: the row max needs one exchange between the wave's halves
//    (v_permlane32_swap), the row sum none;
//  * the key rows fed to the MFMA are permuted inside each 32-key block (bits
//    2 and 3 of the row index swapped), which makes the S^T accumulator
//    registers exactly the B operand of O^T = V^T . P^T: P goes from fp32
//    registers to packed bf16 and straight into the second MFMA;
//  * V^T comes from the cache already tile-transposed, so both LDS operand
//    reads are single 16-byte loads.  LDS rows are padded by one 16-byte chunk
//    (K rows 272 B, V^T rows 144 B): every operand read is a per-lane base plus
//    an immediate, and any 16 consecutive lanes hit 16 distinct bank groups;
//  * the softmax of tile t is interleaved instruction by instruction with the
//    QK^T MFMAs of tile t+1 (sched_group_barrier), and four (six in the
//    fixed-reference kernel's QK^T) LDS operand reads stay in flight ahead of
//    every MFMA;
//  * softmax in the log2 domain (exp2 with log2(e)/sqrt(D) folded into one
//    FMA) against a fixed per-row reference (the row's maximum over tile 0),
//    so no tile needs a maximum or an O rescale; blocks whose probabilities
//    would leave range are flagged and redone by the running-maximum kernel
//    (whose maximum moves only when a tile exceeds it by more than 8).  The
//    row sum is accumulated from the packed bf16 P with v_dot2_f32_bf16, i.e.
//    from the same rounded probabilities the P.V product uses;
//  * key tiles are visited whole tiles first, the few edge tiles of each range
//    (kvc_tiles.hpp) last, so every step but the last two runs without mask
//    code; block-causal attention keeps the logical order and skips the mask
//    on the tiles every row of the block sees;
//  * queries are rotated (3D RoPE, fp32, no FMA) and rounded to bf16 in the
//    prologue, exactly as the cache rotates keys;
//  * workgroup -> (head, query block) mapping is XCD-aware: consecutive
//    blocks of the same head land on the same XCD so they share its L2;
//    block-causal units are dealt longest first, round-robin over the XCDs;
//  * launches with fewer workgroups than CUs split the keys into parts (same
//    kernels, a part index, partial O with its reference and row sum) and
//    merge them in a second pass;
//  * bf16 head_dim 64 has kernels of its own on the same pattern (8-chunk key
//    rows, 4 query fragments, 2 O accumulators, running maximum), and so do
//    its attention-mass scores.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "kvc_common.hip.hpp"
#include "kvc_launch.hpp"
#include "kvc_tiles.hpp"

namespace kvc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// native vector type for 16-byte moves (HIP's uint4 is a class that blocks
// scalar replacement and lands in private memory)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;                       // queries per workgroup
constexpr int kDA = 48, kDB = 80;              // key plane widths for head_dim 128
constexpr int kVTile = 128 * kTile;            // elements of one V^T tile

// swap bits 2 and 3 of a row index inside a 32-row block
__device__ __forceinline__ int perm_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

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
// Two regions' pointers are kept as region 0's address and region 1's offset
// from it, chosen by integer arithmetic: a two-element pointer array chosen by
// a computed region bit becomes an indexed load, which keeps the array in
// scratch memory.
struct RegionPtr {
  uintptr_t p0, d;        // region 0's address, region 1's minus it
  __device__ __forceinline__ void set(const void* a0, const void* a1) {
    p0 = (uintptr_t)a0;
    d = (uintptr_t)a1 - p0;
  }
  template <typename T>
  __device__ __forceinline__ const T* get(int r) const {
    return (const T*)(p0 + (r ? d : (uintptr_t)0));
  }
};

struct TilePtrs {
  RegionPtr k;            // region r, base slot 0, row (tid >> 4)
  RegionPtr v;            // region r, tile 0, piece tid
  int kstride;            // elements per key row of this thread's plane
};

__device__ __forceinline__ TilePtrs tile_ptrs(const KeyRegions& kr, int h, int tid) {
  TilePtrs p;
  const int c = tid & 15;
  p.kstride = c < 6 ? kDA : kDB;
  const uint16_t* k[2];
  const uint16_t* v[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint16_t* plane = c < 6 ? (const uint16_t*)kr.ka[r] + c * 8 : (const uint16_t*)kr.kb[r] + (c - 6) * 8;
    k[r] = plane + ((int64_t)h * kr.cap[r] + (tid >> 4)) * p.kstride;
    v[r] = (const uint16_t*)kr.v[r] + (int64_t)h * (kr.cap[r] / kTile) * kVTile + tid * 8;
  }
  p.k.set(k[0], k[1]);
  p.v.set(v[0], v[1]);
  return p;
}

struct TileRegs {
  u32x4_t k[4];
  u32x4_t v[4];
};

// Rotate this lane's D/2 query elements (row qc, halves hl) and pack them as the
// D/16 B operands of S^T = K . Q^T.
template <int D = 128>
__device__ __forceinline__ void load_query(bf16x8_t* qf, const AttendArgs& a, int h, int qc, int hl) {
  const Geo& g = a.geo;
  const int tok = qc % g.S;
  const int t = a.t0 + qc / g.S, hp = tok / g.grid_w, wp = tok % g.grid_w;
  const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)qc * g.H + h) * D;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
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

// Key of accumulator element i of S^T block kb for lane half hl: kb*32 +
// perm_row((i/4)*8 + hl*4 + i%4), which is kkey(kb, i) + 8*hl with kkey a
// compile-time constant (perm_row moves the hl bit from 2 to 3 and bit 3 of
// (i/4)*8 to 2).  Masks compare kkey against one per-lane bound instead of
// forming 32 key indices.
__device__ __forceinline__ constexpr int kkey(int kb, int i) {
  return kb * 32 + (i & 3) + 4 * ((i >> 2) & 1) + 16 * ((i >> 3) & 1);
}

// keys of the tile outside [lead, nv) get -inf (lead > 0 only in the first tile
// of a range that starts inside a tile)
__device__ __forceinline__ void mask_tile(f32x16_t* s, int lead, int nv, int hl) {
  if (nv >= kBN && lead <= 0) return;
  const int nvh = nv - 8 * hl, leadh = lead - 8 * hl;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (kkey(kb, i) >= nvh || kkey(kb, i) < leadh) s[kb][i] = -INFINITY;
}

// keys of the tile at or past nv get -inf
__device__ __forceinline__ void mask_tile_end(f32x16_t* s, int nv, int hl) {
  if (nv >= kBN) return;
  const int nvh = nv - 8 * hl;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (kkey(kb, i) >= nvh) s[kb][i] = -INFINITY;
}

constexpr float kPLimit = 281474976710656.f;   // 2^48

__device__ __forceinline__ float tile_max(const f32x16_t* sp, float c2) {
  float mt = sp[0][0];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sp[kb][i]);
  return xhalf_max(mt) * c2;
}

// a split-key part's rows: the unnormalised O, the reference m and the row sum
__device__ __forceinline__ void store_partial(const AttendArgs& a, const f32x16_t* o, float m, float lsum, int qrow,
                                              int h, int part, int hl) {
  const float l = xhalf_sum(lsum);
  if (qrow >= a.Lq) return;
  const int64_t r = ((int64_t)part * a.geo.H + h) * a.Lq + qrow;
  float* op = a.split_o + r * 128;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const f32x4_t x = {o[db][gq * 4], o[db][gq * 4 + 1], o[db][gq * 4 + 2], o[db][gq * 4 + 3]};
      *reinterpret_cast<f32x4_t*>(op + db * 32 + gq * 8 + hl * 4) = x;
    }
  if (hl == 0) {
    a.split_ml[r * 2] = m;
    a.split_ml[r * 2 + 1] = l;
  }
}

// the normalised output row; with a.row_m, also the row's normaliser mref + log2(row sum) (mref: the
// reference P was taken against, in log2 units)
template <int D = 128>
__device__ __forceinline__ void store_out(const AttendArgs& a, const f32x16_t* o, float lsum, int qrow, int h, int hl,
                                          float mref) {
  const float l = xhalf_sum(lsum);
  const float inv = 1.f / l;
  if (qrow >= a.Lq) return;
  if (a.row_m != nullptr && hl == 0) a.row_m[(int64_t)h * a.Lq + qrow] = mref + log2f(l);
  uint16_t* op = (uint16_t*)a.out + ((int64_t)qrow * a.geo.H + h) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
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


// ---------------------------------------------------------------------------
// Interleaved pipeline.  LDS rows are padded by one 16-byte chunk (K rows
// 272 B, V^T rows 144 B) instead of XOR-swizzled, so every operand read is a
// per-lane base plus an immediate offset, and any 16 consecutive lanes still
// hit 16 distinct 16-byte bank slots.  Iteration t issues the global loads of
// K(t+2) and V(t+1), then computes S^T(t+1) on the matrix cores interleaved
// instruction by instruction (sched_group_barrier) with the softmax of tile t
// on the VALU; the P.V product of tile t follows.
constexpr int kKSt = 17;                       // K row stride in 16-byte chunks
constexpr int kVSt = 9;                        // V^T row stride in 16-byte chunks
constexpr int kKTileP = kBN * kKSt;            // padded K tile, 16-byte chunks
constexpr int kVTileP = 128 * kVSt;            // padded V^T tile

// S^T for one tile into s, with the softmax of the previous tile (sp) woven in:
// returns P(previous) packed in pb, the tile's row-sum in psum and the scale
// factor alpha for O (1 unless the running max moved).  Scheduling groups ask
// the compiler to emit, per MFMA, one LDS operand read, two exp2 and a few VALU
// operations (FMA, bf16 pack, dot2 sum), so the softmax runs on the VALU while
// the matrix core is busy.
__device__ __forceinline__ void qk_and_softmax(f32x16_t* s, const u32x4_t* lk, const bf16x8_t* qf, int kbase,
                                               const f32x16_t* sp, float& m, float c2, bf16x8_t pb[2][2],
                                               float& psum, float& alpha, bool& upd) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
  float mt = sp[0][0];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sp[kb][i]);
  mt = xhalf_max(mt) * c2;
  upd = mt > m + 8.f;
  const float mn = upd ? mt : m;
  alpha = exp2f(m - mn);
  m = mn;
  const float negm = -m;
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  psum = 0.f;
#pragma unroll
  for (int step = 0; step < 16; ++step) {
    const int kb = step >> 3, ks = step & 7;
    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, lk[kbase + kb * 32 * kKSt + ks * 2]);
    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks], s[kb], 0, 0, 0);
    const int e = step * 2;
    const int pkb = e >> 4, phf = (e >> 3) & 1, pj = e & 7;
    const float p0 = __builtin_amdgcn_exp2f(fmaf(sp[pkb][phf * 8 + pj], c2, negm));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(sp[pkb][phf * 8 + pj + 1], c2, negm));
    const bf16x2_t pr = {(__bf16)p0, (__bf16)p1};
    pb[pkb][phf][pj] = pr[0];
    pb[pkb][phf][pj + 1] = pr[1];
    psum = __builtin_amdgcn_fdot2_f32_bf16(pr, one, psum, false);
  }
  // keep the softmax in this block: without these uses the compiler sinks the
  // exp2s past the caller's rescale branch, away from the MFMAs they should hide
  asm volatile("" ::"v"(psum));
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) asm volatile("" ::"v"(__builtin_bit_cast(u32x4_t, pb[kb][hf])));
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // first operand reads (lookahead)
#pragma unroll
  for (int step = 0; step < 16; ++step) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // next operand read
    __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);   // exp2 x2 (the other VALU work follows its inputs)
  }
}

__device__ __forceinline__ void pv_padded(f32x16_t* o, const u32x4_t* lv, int vbase, bf16x8_t pb[2][2]) {
  // the four accumulators in turn: no MFMA waits for the result of the one before it
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, lv[vbase + db * 32 * kVSt + ks * 2]);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ks >> 1][ks & 1], o[db], 0, 0, 0);
    }
  // keep several V^T operand reads in flight ahead of the MFMAs
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// ---------------------------------------------------------------------------
// v5: v3's interleaved pipeline with 8 waves (256 query rows) per workgroup.
// A 32 KB K+V^T tile is then 16 staging registers per thread instead of 32,
// which leaves the compiler room to keep LDS operand reads in flight; every
// tile loaded to LDS also feeds twice as many query rows (half the L2 traffic
// per query).  Padded LDS rows, double buffered (70 KB), one block per CU.
struct Stage5 {
  u32x4_t k[2];
  u32x4_t v[2];
};

__device__ __forceinline__ void load5(Stage5& st, const TilePtrs& p, int rk, int bk, int rv, int bv) {
  const uint16_t* kp = p.k.get<uint16_t>(rk) + bk * p.kstride;
  const uint16_t* vp = p.v.get<uint16_t>(rv) + (bv / kTile) * kVTile;
#pragma unroll
  for (int i = 0; i < 2; ++i) st.k[i] = *reinterpret_cast<const u32x4_t*>(kp + 32 * i * p.kstride);
#pragma unroll
  for (int i = 0; i < 2; ++i) st.v[i] = *reinterpret_cast<const u32x4_t*>(vp + 4096 * i);
}

__device__ __forceinline__ void store5(const Stage5& st, u32x4_t* lk, u32x4_t* lv, int tid, bool k, bool v) {
  const int c = tid & 15;
  if (k) {
#pragma unroll
    for (int i = 0; i < 2; ++i) lk[((tid >> 4) + 32 * i) * kKSt + c] = st.k[i];
  }
  if (v) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ci = tid + 512 * i;
      lv[(ci >> 3) * kVSt + (ci & 7)] = st.v[i];
    }
  }
}

// With only_flagged set, blocks whose flag is 0 exit at once (the recompute
// pass behind the fixed-reference kernel).  CAUSAL: block-causal attention of
// a clip -- query row r sees the logical key prefix of length
// min(n, (r / causal_block + 1) * causal_block); a workgroup loops only over
// the tiles its longest prefix needs, rows whose prefix ends inside a tile mask
// the rest per lane, and workgroups with the longest prefixes start first.
//
// kparts > 1 (split keys, for launches with fewer workgroups than CUs): the
// tiles are cut into kparts contiguous parts, workgroup (head, part, query
// block) runs over its part only and writes its unnormalised O with the row's
// reference and sum to the split buffers; merge_split_kernel combines them.
template <bool CAUSAL>
__global__ __launch_bounds__(512, 1) void attend_v5_kernel(AttendArgs a, int mblocks, int total, int per_xcd,
                                                           int ntile0, int ntiles, const int32_t* only_flagged,
                                                           int kparts) {
  __shared__ u32x4_t lks[2][kKTileP];
  __shared__ u32x4_t lvs[2][kVTileP];
  const int wg = blockIdx.x;
  // block-causal work per query block grows with the block index: the units are taken longest first,
  // heads minor, one per workgroup in dispatch order, which deals them round-robin over the XCDs, so
  // every XCD gets an equal longest-first share (a contiguous range per XCD would give one XCD the heavy
  // half of a head and another its light half)
  const int lin = CAUSAL ? wg : (wg & 7) * per_xcd + (wg >> 3);
  if (lin >= total) return;
  if (only_flagged != nullptr && only_flagged[lin] == 0) return;
  const int hp = CAUSAL ? lin % a.geo.H : lin / mblocks;   // head * kparts + part (kparts = 1 when causal)
  const int h = hp / kparts, part = hp - h * kparts;
  const int mb = CAUSAL ? mblocks - 1 - lin / a.geo.H : lin - hp * mblocks;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int qrow = mb * 256 + wave * 32 + l32;
  // not causal: edges-last order, as in the fixed-reference kernel (a split part covers the same tiles in both)
  TileSeq ts = CAUSAL ? tile_seq(a.keys, ntile0, ntiles) : tile_seq_edges_last(a.keys, ntile0, ntiles);
  // balanced parts: [part * ntiles / kparts, (part + 1) * ntiles / kparts), never empty (kparts <= ntiles / 4)
  ts.first = part * ntiles / kparts;
  const int kbase = perm_row(l32) * kKSt + hl;
  const int vbase = l32 * kVSt + hl;
  int nt = (part + 1) * ntiles / kparts - ts.first, lim = 0, lim_lo = 0;
  if (CAUSAL) {
    const int cb = a.causal_block, nall = a.keys.n[0] + a.keys.n[1];
    auto limit = [&](int r) { return min(nall, (r / cb + 1) * cb); };
    const int r0 = mb * 256, r1 = min(a.Lq, r0 + 256) - 1;
    lim_lo = limit(r0);
    lim = limit(min(qrow, a.Lq - 1));
    const int lim_hi = limit(r1), n0 = a.keys.n[0];
    nt = lim_hi <= n0 ? (lim_hi + kBN - 1) / kBN : ntile0 + (lim_hi - n0 + kBN - 1) / kBN;
  }
  const int last = nt - 1;
  // mask tile t: slots past the region's valid prefix, and (causal) keys past this row's prefix
  auto mask = [&](f32x16_t* s, int t) {
    const int nv = CAUSAL ? ts.valid_w(t) : ts.valid(t);   // causal: logical order
    if (CAUSAL) {
      const int lb = t < ntile0 ? t * kBN : a.keys.n[0] + (t - ntile0) * kBN;
      if (lb + kBN > lim_lo) {
        mask_tile_end(s, min(nv, lim - lb), hl);
        return;
      }
    }
    mask_tile(s, CAUSAL ? ts.lead_w(t) : ts.lead(t), nv, hl);
  };
  // tile lookups of the prologue (logical order when causal)
  auto reg = [&](int t) { return CAUSAL ? ts.region_w(t) : ts.region(t); };
  auto bas = [&](int t) { return CAUSAL ? ts.base_w(t) : ts.base(t); };
  const TilePtrs tp = tile_ptrs(a.keys, h, tid);

  Stage5 st;
  load5(st, tp, reg(0), bas(0), reg(0), bas(0));
  bf16x8_t qf[8];
  load_query(qf, a, h, min(qrow, a.Lq - 1), hl);
  store5(st, lks[0], lvs[0], tid, true, true);
  {
    const int t1 = min(1, last);
    load5(st, tp, reg(t1), bas(t1), 0, 0);
    store5(st, lks[1], lvs[1], tid, true, false);
  }
  f32x16_t o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  const float c2 = a.scale * 1.4426950408889634f;
  __syncthreads();
  f32x16_t sa[2], sb[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sa[kb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, lks[0][kbase + kb * 32 * kKSt + ks * 2]);
      sa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks], sa[kb], 0, 0, 0);
    }
  }
  mask(sa, 0);
  __syncthreads();   // every wave has read K(0) before step 0 stores K(2) over it

  auto step = [&](int t, f32x16_t* scur, f32x16_t* snext) {
    const int tk = min(t + 2, last), tv = min(t + 1, last);
    load5(st, tp, CAUSAL ? ts.region_w(tk) : ts.region(tk), CAUSAL ? ts.base_w(tk) : ts.base(tk),
          CAUSAL ? ts.region_w(tv) : ts.region(tv), CAUSAL ? ts.base_w(tv) : ts.base(tv));
    bf16x8_t pb[2][2];
    float psum, alpha;
    bool upd;
    qk_and_softmax(snext, lks[(t + 1) & 1], qf, kbase, scur, m, c2, pb, psum, alpha, upd);
    if (__ballot(upd) != 0) {
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[d][i] *= alpha;
    }
    lsum = lsum * alpha + psum;
    pv_padded(o, lvs[t & 1], vbase, pb);
    mask(snext, min(t + 1, last));
    store5(st, lks[t & 1], lvs[(t + 1) & 1], tid, true, true);
    __syncthreads();
  };

  int t = 0;
  for (; t + 1 < nt; t += 2) {
    step(t, sa, sb);
    step(t + 1, sb, sa);
  }
  if (t < nt) step(t, sa, sb);
  if (kparts > 1)
    store_partial(a, o, m, lsum, qrow, h, part, hl);
  else
    store_out(a, o, lsum, qrow, h, hl, m);
}

// ---------------------------------------------------------------------------
// bf16, head_dim 64: the running-maximum pipeline above at half the head
// width.  A stored key is 8 chunks of 16 bytes (3 of the KA plane, dims 0..23,
// then 5 of the KB plane) and a V^T tile 64 rows of 8 chunks, so each of the
// 512 threads stages one chunk of each per 64-key tile; a lane holds 4 query
// fragments and two O accumulators.  Per tile a wave issues 8 MFMAs for S^T
// and 8 for P.V beside the 32 exponentials of the previous tile.  Keys must be
// stored rotated (raw-key caches of this width take the general kernel).
constexpr int kD64A = 24, kD64B = 40;          // key plane widths for head_dim 64
constexpr int kK64St = 9;                      // K row stride in 16-byte chunks (8 + pad)
constexpr int kV64St = 9;                      // V^T row stride in 16-byte chunks (8 + pad)
constexpr int kV64Tile = 64 * kTile;           // elements of one V^T tile

// Thread tid moves chunk (tid & 7) of K row (tid >> 3) and the 16-byte piece tid of the V^T tile.
struct Tile64Ptrs {
  RegionPtr k;
  RegionPtr v;
  int kstride;
};

__device__ __forceinline__ Tile64Ptrs tile64_ptrs(const KeyRegions& kr, int h, int tid) {
  Tile64Ptrs p;
  const int c = tid & 7;
  p.kstride = c < 3 ? kD64A : kD64B;
  const uint16_t* k[2];
  const uint16_t* v[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint16_t* plane = c < 3 ? (const uint16_t*)kr.ka[r] + c * 8 : (const uint16_t*)kr.kb[r] + (c - 3) * 8;
    k[r] = plane + ((int64_t)h * kr.cap[r] + (tid >> 3)) * p.kstride;
    v[r] = (const uint16_t*)kr.v[r] + (int64_t)h * (kr.cap[r] / kTile) * kV64Tile + tid * 8;
  }
  p.k.set(k[0], k[1]);
  p.v.set(v[0], v[1]);
  return p;
}

struct Stage64 {
  u32x4_t k, v;
};

__device__ __forceinline__ void load64(Stage64& st, const Tile64Ptrs& p, int rk, int bk, int rv, int bv) {
  st.k = *reinterpret_cast<const u32x4_t*>(p.k.get<uint16_t>(rk) + bk * p.kstride);
  st.v = *reinterpret_cast<const u32x4_t*>(p.v.get<uint16_t>(rv) + (bv / kTile) * kV64Tile);
}

__device__ __forceinline__ void store64(const Stage64& st, u32x4_t* lk, u32x4_t* lv, int tid, bool v) {
  lk[(tid >> 3) * kK64St + (tid & 7)] = st.k;
  if (v) lv[(tid >> 3) * kV64St + (tid & 7)] = st.v;
}

// S^T of one tile (8 MFMAs) with the running-maximum softmax of the previous tile woven in, four
// elements per MFMA; P packed as in the head_dim-128 kernel.
__device__ __forceinline__ void qk_and_softmax64(f32x16_t* s, const u32x4_t* lk, const bf16x8_t* qf, int kbase,
                                                 const f32x16_t* sp, float& m, float c2, bf16x8_t pb[2][2],
                                                 float& psum, float& alpha, bool& upd) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
  const float mt = tile_max(sp, c2);
  upd = mt > m + 8.f;
  const float mn = upd ? mt : m;
  alpha = exp2f(m - mn);
  m = mn;
  const float negm = -m;
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  psum = 0.f;
#pragma unroll
  for (int step = 0; step < 8; ++step) {
    const int kb = step >> 2, ks = step & 3;
    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, lk[kbase + kb * 32 * kK64St + ks * 2]);
    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks], s[kb], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const int e = step * 4 + j;
      const int pkb = e >> 4, phf = (e >> 3) & 1, pj = e & 7;
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sp[pkb][phf * 8 + pj], c2, negm));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sp[pkb][phf * 8 + pj + 1], c2, negm));
      const bf16x2_t pr = {(__bf16)p0, (__bf16)p1};
      pb[pkb][phf][pj] = pr[0];
      pb[pkb][phf][pj + 1] = pr[1];
      psum = __builtin_amdgcn_fdot2_f32_bf16(pr, one, psum, false);
    }
  }
  asm volatile("" ::"v"(psum));
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) asm volatile("" ::"v"(__builtin_bit_cast(u32x4_t, pb[kb][hf])));
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // first operand reads (lookahead)
#pragma unroll
  for (int step = 0; step < 8; ++step) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // next operand read
    __builtin_amdgcn_sched_group_barrier(0x400, 4, 0);   // exp2 x4
  }
}

__device__ __forceinline__ void pv64(f32x16_t* o, const u32x4_t* lv, int vbase, bf16x8_t pb[2][2]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, lv[vbase + db * 32 * kV64St + ks * 2]);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ks >> 1][ks & 1], o[db], 0, 0, 0);
    }
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

template <bool CAUSAL>
__global__ __launch_bounds__(512, 1) void attend_d64_kernel(AttendArgs a, int mblocks, int total, int per_xcd,
                                                            int ntile0, int ntiles) {
  __shared__ u32x4_t lks[2][kBN * kK64St];
  __shared__ u32x4_t lvs[2][64 * kV64St];
  const int wg = blockIdx.x;
  // unit order as in the head_dim-128 kernels (block-causal: longest first, round-robin over the XCDs)
  const int lin = CAUSAL ? wg : (wg & 7) * per_xcd + (wg >> 3);
  if (lin >= total) return;
  const int h = CAUSAL ? lin % a.geo.H : lin / mblocks;
  const int mb = CAUSAL ? mblocks - 1 - lin / a.geo.H : lin - h * mblocks;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int qrow = mb * 256 + wave * 32 + l32;
  const TileSeq ts = CAUSAL ? tile_seq(a.keys, ntile0, ntiles) : tile_seq_edges_last(a.keys, ntile0, ntiles);
  const int kbase = perm_row(l32) * kK64St + hl;
  const int vbase = l32 * kV64St + hl;
  int nt = ntiles, lim = 0, lim_lo = 0;
  if (CAUSAL) {
    const int cb = a.causal_block, nall = a.keys.n[0] + a.keys.n[1];
    auto limit = [&](int r) { return min(nall, (r / cb + 1) * cb); };
    const int r0 = mb * 256, r1 = min(a.Lq, r0 + 256) - 1;
    lim_lo = limit(r0);
    lim = limit(min(qrow, a.Lq - 1));
    const int lim_hi = limit(r1), n0 = a.keys.n[0];
    nt = lim_hi <= n0 ? (lim_hi + kBN - 1) / kBN : ntile0 + (lim_hi - n0 + kBN - 1) / kBN;
  }
  const int last = nt - 1;
  auto mask = [&](f32x16_t* sv, int t) {
    const int nv = CAUSAL ? ts.valid_w(t) : ts.valid(t);
    if (CAUSAL) {
      const int lb = t < ntile0 ? t * kBN : a.keys.n[0] + (t - ntile0) * kBN;
      if (lb + kBN > lim_lo) {
        mask_tile_end(sv, min(nv, lim - lb), hl);
        return;
      }
    }
    mask_tile(sv, CAUSAL ? ts.lead_w(t) : ts.lead(t), nv, hl);
  };
  auto reg = [&](int t) { return CAUSAL ? ts.region_w(t) : ts.region(t); };
  auto bas = [&](int t) { return CAUSAL ? ts.base_w(t) : ts.base(t); };
  const Tile64Ptrs tp = tile64_ptrs(a.keys, h, tid);

  Stage64 st;
  load64(st, tp, reg(0), bas(0), reg(0), bas(0));
  bf16x8_t qf[4];
  load_query<64>(qf, a, h, min(qrow, a.Lq - 1), hl);
  store64(st, lks[0], lvs[0], tid, true);
  {
    const int t1 = min(1, last);
    load64(st, tp, reg(t1), bas(t1), 0, 0);
    store64(st, lks[1], lvs[1], tid, false);
  }
  f32x16_t o[2];
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  const float c2 = a.scale * 1.4426950408889634f;
  __syncthreads();
  f32x16_t sa[2], sb[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sa[kb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, lks[0][kbase + kb * 32 * kK64St + ks * 2]);
      sa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks], sa[kb], 0, 0, 0);
    }
  }
  mask(sa, 0);
  __syncthreads();   // every wave has read K(0) before step 0 stores K(2) over it

  // step t: S^T(t+1) beside the softmax of tile t, then P(t).V(t); K(t+2) and V(t+1) staged meanwhile
  auto step = [&](int t, f32x16_t* scur, f32x16_t* snext) {
    const int tk = min(t + 2, last), tv = min(t + 1, last);
    load64(st, tp, reg(tk), bas(tk), reg(tv), bas(tv));
    bf16x8_t pb[2][2];
    float psum, alpha;
    bool upd;
    qk_and_softmax64(snext, lks[(t + 1) & 1], qf, kbase, scur, m, c2, pb, psum, alpha, upd);
    if (__ballot(upd) != 0) {
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[d][i] *= alpha;
    }
    lsum = lsum * alpha + psum;
    pv64(o, lvs[t & 1], vbase, pb);
    mask(snext, min(t + 1, last));
    store64(st, lks[t & 1], lvs[(t + 1) & 1], tid, true);
    __syncthreads();
  };
  int t = 0;
  for (; t + 1 < nt; t += 2) {
    step(t, sa, sb);
    step(t + 1, sb, sa);
  }
  if (t < nt) step(t, sa, sb);
  store_out<64>(a, o, lsum, qrow, h, hl, m);
}

// out = (sum_s 2^(m_s - M) O_s) / (sum_s 2^(m_s - M) l_s) over the key parts,
// M = max_s m_s; one thread per (head, row, 4 dims).
__global__ __launch_bounds__(256) void merge_split_kernel(AttendArgs a, int kparts) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int c = (int)(id & 31);
  const int64_t hr = id >> 5;
  if (hr >= (int64_t)a.geo.H * a.Lq) return;
  const int h = (int)(hr / a.Lq), row = (int)(hr - (int64_t)h * a.Lq);
  float M = -INFINITY;
  for (int p = 0; p < kparts; ++p) M = fmaxf(M, a.split_ml[(((int64_t)p * a.geo.H + h) * a.Lq + row) * 2]);
  float l = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < kparts; ++p) {
    const int64_t r = ((int64_t)p * a.geo.H + h) * a.Lq + row;
    const float w = __builtin_amdgcn_exp2f(a.split_ml[r * 2] - M);
    l += w * a.split_ml[r * 2 + 1];
    const f32x4_t x = *reinterpret_cast<const f32x4_t*>(a.split_o + r * 128 + c * 4);
    acc += w * x;
  }
  const float inv = 1.f / l;
  if (a.row_m != nullptr && c == 0) a.row_m[(int64_t)h * a.Lq + row] = M + log2f(l);
  union {
    uint2 u;
    __bf16 b[4];
  } y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y.b[e] = (__bf16)(acc[e] * inv);
  *reinterpret_cast<uint2*>((uint16_t*)a.out + ((int64_t)row * a.geo.H + h) * 128 + c * 4) = y.u;
}

// ---------------------------------------------------------------------------
// Attention-mass scores on the matrix cores (bf16, head_dim 128; head_dim 64
// further below).  The query
// window arrives already rotated and rounded (qbf: [H][Nq][128] bf16).
//
// Rows pass: per (head, query) the softmax normaliser over every valid key,
// folded into one log2-domain constant  M = m + log2(l)  with
// m = max_j c2 s_j and l = sum_j exp2(c2 s_j - m), c2 = log2(e)/sqrt(D); the
// probability of key j is then exp2(c2 s_j - M).  It runs on the attention
// kernel's 8-wave pipeline with a fixed per-row reference (m = the row's
// maximum over its first key tile; blocks whose sums leave range are flagged
// and redone by a 4-wave running-maximum kernel), S^T = K.Q^T per 64-key tile
// as in attention, no P.V.
//
// Columns pass: per (head, key) the sum over queries of exp2(c2 s - M).
// S = Q.K^T with the lane owning one key column: workgroup = 4 waves x 32
// keys of one region, their K fragments held in registers; query tiles of 32
// rows (and their M) stream through LDS, double buffered; each lane sums its
// 16 rows of every tile, and the two wave halves are added at the end.

__device__ __forceinline__ void tile_load_k(TileRegs& tr, const TilePtrs& p, int r, int base) {
  const uint16_t* kp = p.k.get<uint16_t>(r) + base * p.kstride;
#pragma unroll
  for (int i = 0; i < 4; ++i) tr.k[i] = *reinterpret_cast<const u32x4_t*>(kp + 16 * i * p.kstride);
}

__device__ __forceinline__ void tile_store_k_padded(const TileRegs& tr, u32x4_t* lk, int tid) {
  const int c = tid & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) lk[((tid >> 4) + 16 * i) * kKSt + c] = tr.k[i];
}

// The running-maximum rows pass (4 waves x 32 rows).  It recomputes the rows
// of the 256-row blocks the fixed-reference pass flagged: flags[h * mb256 +
// mb / 2] for its 128-row block (h, mb).
__global__ __launch_bounds__(256, 2) void score_rows_mfma_kernel(ScoreArgs a, const uint16_t* qbf, int mblocks,
                                                                 int total, int ntile0, int ntiles, int mb256) {
  __shared__ u32x4_t lks[2][kKTileP];
  const int lin = blockIdx.x;
  if (lin >= total) return;
  const int h = lin / mblocks;
  const int mb = lin - h * mblocks;
  if (a.flags[h * mb256 + mb / 2] == 0) return;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int qrow = mb * kBM + wave * 32 + l32;
  const TileSeq ts = tile_seq(a.keys, ntile0, ntiles);
  const int kbase = perm_row(l32) * kKSt + hl;
  const TilePtrs tp = tile_ptrs(a.keys, h, tid);

  TileRegs tr;
  tile_load_k(tr, tp, ts.region(0), ts.base(0));
  bf16x8_t qf[8];
  {
    const uint16_t* qp = qbf + ((int64_t)h * a.Nq + min(qrow, a.Nq - 1)) * 128 + hl * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(qp + ks * 16));
  }
  tile_store_k_padded(tr, lks[0], tid);
  __syncthreads();
  const float c2 = a.scale * 1.4426950408889634f;
  float m = -INFINITY, l = 0.f;
  for (int t = 0; t < ntiles; ++t) {
    const bool more = t + 1 < ntiles;
    if (more) tile_load_k(tr, tp, ts.region(t + 1), ts.base(t + 1));
    f32x16_t sc[2];
    const u32x4_t* lk = lks[t & 1];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, lk[kbase + kb * 32 * kKSt + ks * 2]),
                                                         qf[ks], sc[kb], 0, 0, 0);
    }
    mask_tile(sc, ts.lead(t), ts.valid(t), hl);
    float mt = sc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sc[kb][i]);
    const float mn = fmaxf(m, xhalf_max(mt) * c2);
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) ps += __builtin_amdgcn_exp2f(fmaf(sc[kb][i], c2, -mn));
    l = l * __builtin_amdgcn_exp2f(m - mn) + ps;
    m = mn;
    if (more) tile_store_k_padded(tr, lks[(t + 1) & 1], tid);
    __syncthreads();
  }
  const float lt = xhalf_sum(l);
  if (hl == 0 && qrow < a.Nq) a.m[(int64_t)h * a.Nq + qrow] = m + log2f(lt);
}

// Rows pass on the 8-wave pipeline (the fixed-reference attention kernel
// without P.V): 256 query rows per workgroup, key tiles staged in LDS double
// buffered, S^T(t+1) on the matrix cores interleaved with the exponentials of
// S^T(t) against a fixed per-row reference (the row's maximum over tile 0), so
// no tile needs a maximum.  M = ref + log2(sum); a workgroup whose partial sums
// leave range (or turn non-finite) sets its flag, and the running-maximum pass
// redoes its rows.
__device__ __forceinline__ void qk_and_sum(f32x16_t* s, const u32x4_t* lk, const bf16x8_t* qf, int kbase,
                                           const f32x16_t* sp, float negm, float c2, float& psum) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
  float p0s = 0.f, p1s = 0.f;
#pragma unroll
  for (int step = 0; step < 16; ++step) {
    const int kb = step & 1, ks = step >> 1;      // the two accumulators alternate
    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, lk[kbase + kb * 32 * kKSt + ks * 2]);
    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks], s[kb], 0, 0, 0);
    const int e = step * 2;
    const int pkb = e >> 4, pi = e & 15;
    p0s += __builtin_amdgcn_exp2f(fmaf(sp[pkb][pi], c2, negm));
    p1s += __builtin_amdgcn_exp2f(fmaf(sp[pkb][pi + 1], c2, negm));
  }
  psum = p0s + p1s;
  asm volatile("" ::"v"(psum));
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // operand reads ahead
#pragma unroll
  for (int step = 0; step < 16; ++step) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // next operand read
    __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);   // exp2 x2
  }
}

__global__ __launch_bounds__(512, 1) void score_rows_v5f_kernel(ScoreArgs a, const uint16_t* qbf, int mblocks,
                                                                int total, int per_xcd, int ntile0, int ntiles) {
  __shared__ u32x4_t lks[2][kKTileP];
  __shared__ int s_flag;
  const int wg = blockIdx.x;
  const int lin = (wg & 7) * per_xcd + (wg >> 3);       // consecutive blocks of a head on one XCD
  if (lin >= total) return;
  const int h = lin / mblocks, mb = lin - (lin / mblocks) * mblocks;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int qrow = mb * 256 + wave * 32 + l32;
  const TileSeq ts = tile_seq_edges_last(a.keys, ntile0, ntiles);
  const int kbase = perm_row(l32) * kKSt + hl;
  const int nt = ntiles, last = nt - 1;
  const TilePtrs tp = tile_ptrs(a.keys, h, tid);
  if (tid == 0) s_flag = 0;
  const int c = tid & 15;
  auto load_k = [&](u32x4_t* st, int r, int base) {
    const uint16_t* kp = tp.k.get<uint16_t>(r) + base * tp.kstride;
#pragma unroll
    for (int i = 0; i < 2; ++i) st[i] = *reinterpret_cast<const u32x4_t*>(kp + 32 * i * tp.kstride);
  };
  auto store_k = [&](const u32x4_t* st, u32x4_t* lk) {
#pragma unroll
    for (int i = 0; i < 2; ++i) lk[((tid >> 4) + 32 * i) * kKSt + c] = st[i];
  };
  u32x4_t st[2];
  load_k(st, ts.region(0), ts.base(0));
  bf16x8_t qf[8];
  {
    const uint16_t* qp = qbf + ((int64_t)h * a.Nq + min(qrow, a.Nq - 1)) * 128 + hl * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(qp + ks * 16));
  }
  store_k(st, lks[0]);
  {
    const int t1 = min(1, last);
    load_k(st, ts.region(t1), ts.base(t1));
    store_k(st, lks[1]);
  }
  __syncthreads();
  const float c2 = a.scale * 1.4426950408889634f;
  f32x16_t sa[2], sb[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sa[kb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      sa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, lks[0][kbase + kb * 32 * kKSt + ks * 2]),
                                                       qf[ks], sa[kb], 0, 0, 0);
  }
  mask_tile(sa, ts.lead(0), ts.valid(0), hl);
  const float negm = -tile_max(sa, c2);       // tile 0 holds a valid key for every row
  float lsum = 0.f, pmax = 0.f;
  __syncthreads();                            // every wave has read K(0) before step 0 stores K(2) there
  auto step = [&](int t, f32x16_t* scur, f32x16_t* snext, auto masked) {
    const int tk = min(t + 2, last);
    constexpr bool any = decltype(masked)::value;
    load_k(st, any ? ts.region(tk) : ts.region_w(tk), any ? ts.base(tk) : ts.base_w(tk));
    float psum;
    qk_and_sum(snext, lks[(t + 1) & 1], qf, kbase, scur, negm, c2, psum);
    pmax = fmaxf(pmax, psum);
    lsum += psum;
    if constexpr (decltype(masked)::value) {
      const int tn = min(t + 1, last);
      mask_tile(snext, ts.lead(tn), ts.valid(tn), hl);
    }
    store_k(st, lks[t & 1]);
    __syncthreads();
  };
  using Masked = std::integral_constant<bool, true>;
  using Clean = std::integral_constant<bool, false>;
  const int clean = max(0, ts.whole_prefix(nt) - 2);
  int t = 0;
  for (; t + 1 < clean; t += 2) {
    step(t, sa, sb, Clean{});
    step(t + 1, sb, sa, Clean{});
  }
  for (; t + 1 < nt; t += 2) {
    step(t, sa, sb, Masked{});
    step(t + 1, sb, sa, Masked{});
  }
  if (t < nt) step(t, sa, sb, Masked{});   // step t sums tile t (the last step's S^T(t + 1) is unused)
  if (__ballot(!(pmax <= kPLimit)) != 0 && lane == 0) s_flag = 1;
  __syncthreads();
  if (tid == 0) a.flags[lin] = s_flag;
  const float l = xhalf_sum(lsum);
  if (hl == 0 && qrow < a.Nq) a.m[(int64_t)h * a.Nq + qrow] = -negm + log2f(l);
}

constexpr int kQT = 32;                          // query rows per columns-pass tile

__global__ __launch_bounds__(256, 2) void score_cols_mfma_kernel(ScoreArgs a, const uint16_t* qbf, int region,
                                                                 int kblocks, int total) {
  __shared__ u32x4_t lq[2][kQT * kKSt];
  __shared__ __attribute__((aligned(16))) float lm[2][kQT];
  const int lin = blockIdx.x;
  if (lin >= total) return;
  const int h = lin / kblocks;
  const int kblk = lin - h * kblocks;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int nk = a.keys.n[region];
  const int key = kblk * 128 + wave * 32 + l32;
  // this lane's key column: B operand fragments of S = Q.K^T
  bf16x8_t kf[8];
  {
    const int kk = min(key, nk - 1);
    const int64_t row = (int64_t)h * a.keys.cap[region] + kk;
    const uint16_t* ka = (const uint16_t*)a.keys.ka[region] + row * kDA;
    const uint16_t* kb = (const uint16_t*)a.keys.kb[region] + row * kDB;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int d = ks * 16 + hl * 8;
      const uint16_t* src = d < kDA ? ka + d : kb + (d - kDA);
      kf[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(src));
    }
  }
  const int nqt = (a.Nq + kQT - 1) / kQT;
  const uint16_t* qh = qbf + (int64_t)h * a.Nq * 128;
  const float* mrow = a.m + (int64_t)h * a.Nq;
  // thread tid stages chunks tid and tid + 256 of a 32 x 16-chunk query tile
  auto load_q = [&](int qt, u32x4_t* st, float& mv) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ci = tid + 256 * i;
      const int r = min(qt * kQT + (ci >> 4), a.Nq - 1);
      st[i] = *reinterpret_cast<const u32x4_t*>(qh + (int64_t)r * 128 + (ci & 15) * 8);
    }
    if (tid < kQT) {
      const int r = qt * kQT + tid;
      mv = r < a.Nq ? mrow[r] : INFINITY;   // rows past the window contribute exp2(-inf) = 0
    }
  };
  auto store_q = [&](int buf, const u32x4_t* st, float mv) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ci = tid + 256 * i;
      lq[buf][(ci >> 4) * kKSt + (ci & 15)] = st[i];
    }
    if (tid < kQT) lm[buf][tid] = mv;
  };
  u32x4_t st[2];
  float mv = 0.f;
  load_q(0, st, mv);
  store_q(0, st, mv);
  __syncthreads();
  const float c2 = a.scale * 1.4426950408889634f;
  const int qbase = l32 * kKSt + hl;
  float acc = 0.f;
  for (int qt = 0; qt < nqt; ++qt) {
    const bool more = qt + 1 < nqt;
    if (more) load_q(qt + 1, st, mv);
    const u32x4_t* q = lq[qt & 1];
    f32x16_t c;
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, q[qbase + ks * 2]), kf[ks], c, 0, 0, 0);
    // accumulator i is query row (i/4)*8 + hl*4 + i%4 of the tile
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const float4 mg = *reinterpret_cast<const float4*>(&lm[qt & 1][g4 * 8 + hl * 4]);
      acc += __builtin_amdgcn_exp2f(fmaf(c[g4 * 4 + 0], c2, -mg.x));
      acc += __builtin_amdgcn_exp2f(fmaf(c[g4 * 4 + 1], c2, -mg.y));
      acc += __builtin_amdgcn_exp2f(fmaf(c[g4 * 4 + 2], c2, -mg.z));
      acc += __builtin_amdgcn_exp2f(fmaf(c[g4 * 4 + 3], c2, -mg.w));
    }
    if (more) store_q((qt + 1) & 1, st, mv);
    __syncthreads();
  }
  const float tot = xhalf_sum(acc);
  if (hl == 0 && key < nk) {
    const int ncap = a.keys.cap[0] + a.keys.cap[1];
    const int p = region == 0 ? key : a.keys.cap[0] + key;
    a.part[(int64_t)h * ncap + p] = tot;
  }
}

// Rows pass: the fixed-reference 8-wave kernel, then the running-maximum kernel
// on the flagged blocks only; then the columns pass.
hipError_t launch_score_mfma(const ScoreArgs& a, const uint16_t* qbf, hipStream_t s) {
  const int mblocks = (a.Nq + kBM - 1) / kBM;
  const int mb256 = (a.Nq + 255) / 256;
  const int ntile0 = range_tiles(a.keys, 0);
  const int ntile1 = range_tiles(a.keys, 1);
  ScoreArgs b = a;
  int n0 = ntile0, nt = ntile0 + ntile1;
  if (ntile0 == 0) {   // keep region 0 non-empty for the tile sequence
    b.keys.ka[0] = a.keys.ka[1];
    b.keys.kb[0] = a.keys.kb[1];
    b.keys.v[0] = a.keys.v[1];
    b.keys.t[0] = a.keys.t[1];
    b.keys.cap[0] = a.keys.cap[1];
    b.keys.lo[0] = a.keys.lo[1];
    b.keys.n[0] = a.keys.n[1];
    b.keys.lo[1] = 0;
    b.keys.n[1] = 0;
    n0 = ntile1;
    nt = ntile1;
  }
  if (nt == 0 || a.Nq == 0) return hipSuccess;
  if (!a.rows_given) {   // else a.m holds the attention's row normalisers
    const int total256 = mb256 * a.geo.H, per_xcd = (total256 + 7) / 8;
    hipLaunchKernelGGL(score_rows_v5f_kernel, dim3(8 * per_xcd), dim3(512), 0, s, b, qbf, mb256, total256, per_xcd,
                       n0, nt);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    const int total = mblocks * a.geo.H;
    hipLaunchKernelGGL(score_rows_mfma_kernel, dim3(total), dim3(256), 0, s, b, qbf, mblocks, total, n0, nt, mb256);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  // columns: original region numbering (part is indexed by physical slot).  The 4-wave kernel stays: an
  // 8-wave version with 128-row query stages (201 VGPRs, one workgroup per CU) was 10 % slower.
  for (int r = 0; r < 2; ++r) {
    if (a.keys.n[r] == 0) continue;
    const int kblocks = (a.keys.n[r] + 127) / 128;
    const int tot = kblocks * a.geo.H;
    hipLaunchKernelGGL(score_cols_mfma_kernel, dim3(tot), dim3(256), 0, s, a, qbf, r, kblocks, tot);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Scores for bf16 head_dim 64 (key rows of 8 chunks: 3 of the KA plane, 5 of
// the KB plane).  Rows pass: 4 waves x 32 query rows, 64-key tiles double
// buffered in LDS, running maximum, every block (no flags).  Columns pass: as
// for head_dim 128, a lane's key column held in registers (4 fragments), query
// tiles of 32 rows (one 16-byte chunk per thread) streamed through LDS.
__global__ __launch_bounds__(256, 2) void score_rows_d64_kernel(ScoreArgs a, const uint16_t* qbf, int mblocks,
                                                                int total, int ntile0, int ntiles) {
  __shared__ u32x4_t lks[2][kBN * kK64St];
  const int lin = blockIdx.x;
  if (lin >= total) return;
  const int h = lin / mblocks;
  const int mb = lin - h * mblocks;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int qrow = mb * kBM + wave * 32 + l32;
  const TileSeq ts = tile_seq(a.keys, ntile0, ntiles);
  const int kbase = perm_row(l32) * kK64St + hl;
  const Tile64Ptrs tp = tile64_ptrs(a.keys, h, tid);   // rows (tid >> 3) and (tid >> 3) + 32 of a tile
  auto load_k = [&](u32x4_t* st, int r, int base) {
    const uint16_t* kp = tp.k.get<uint16_t>(r) + base * tp.kstride;
#pragma unroll
    for (int i = 0; i < 2; ++i) st[i] = *reinterpret_cast<const u32x4_t*>(kp + 32 * i * tp.kstride);
  };
  auto store_k = [&](const u32x4_t* st, u32x4_t* lk) {
#pragma unroll
    for (int i = 0; i < 2; ++i) lk[((tid >> 3) + 32 * i) * kK64St + (tid & 7)] = st[i];
  };
  u32x4_t st[2];
  load_k(st, ts.region(0), ts.base(0));
  bf16x8_t qf[4];
  {
    const uint16_t* qp = qbf + ((int64_t)h * a.Nq + min(qrow, a.Nq - 1)) * 64 + hl * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(qp + ks * 16));
  }
  store_k(st, lks[0]);
  __syncthreads();
  const float c2 = a.scale * 1.4426950408889634f;
  float m = -INFINITY, l = 0.f;
  for (int t = 0; t < ntiles; ++t) {
    const bool more = t + 1 < ntiles;
    if (more) load_k(st, ts.region(t + 1), ts.base(t + 1));
    f32x16_t sc[2];
    const u32x4_t* lk = lks[t & 1];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, lk[kbase + kb * 32 * kK64St + ks * 2]),
                                                         qf[ks], sc[kb], 0, 0, 0);
    }
    mask_tile(sc, ts.lead(t), ts.valid(t), hl);
    // tile 0 (logical order) holds a valid key, so m is finite from the first tile on
    const float mn = fmaxf(m, tile_max(sc, c2));
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) ps += __builtin_amdgcn_exp2f(fmaf(sc[kb][i], c2, -mn));
    l = l * __builtin_amdgcn_exp2f(m - mn) + ps;
    m = mn;
    if (more) store_k(st, lks[(t + 1) & 1]);
    __syncthreads();
  }
  const float lt = xhalf_sum(l);
  if (hl == 0 && qrow < a.Nq) a.m[(int64_t)h * a.Nq + qrow] = m + log2f(lt);
}

__global__ __launch_bounds__(256, 2) void score_cols_d64_kernel(ScoreArgs a, const uint16_t* qbf, int region,
                                                                int kblocks, int total) {
  constexpr int kQT64 = 32;                      // query rows per tile
  __shared__ u32x4_t lq[2][kQT64 * kK64St];
  __shared__ __attribute__((aligned(16))) float lm[2][kQT64];
  const int lin = blockIdx.x;
  if (lin >= total) return;
  const int h = lin / kblocks;
  const int kblk = lin - h * kblocks;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int nk = a.keys.n[region];
  const int key = kblk * 128 + wave * 32 + l32;
  bf16x8_t kf[4];
  {
    const int kk = min(key, nk - 1);
    const int64_t row = (int64_t)h * a.keys.cap[region] + kk;
    const uint16_t* ka = (const uint16_t*)a.keys.ka[region] + row * kD64A;
    const uint16_t* kb = (const uint16_t*)a.keys.kb[region] + row * kD64B;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int d = ks * 16 + hl * 8;
      const uint16_t* src = d < kD64A ? ka + d : kb + (d - kD64A);
      kf[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(src));
    }
  }
  const int nqt = (a.Nq + kQT64 - 1) / kQT64;
  const uint16_t* qh = qbf + (int64_t)h * a.Nq * 64;
  const float* mrow = a.m + (int64_t)h * a.Nq;
  // thread tid stages chunk (tid & 7) of tile row (tid >> 3), and threads 0..31 the rows' M
  auto load_q = [&](int qt, u32x4_t& st, float& mv) {
    const int r = min(qt * kQT64 + (tid >> 3), a.Nq - 1);
    st = *reinterpret_cast<const u32x4_t*>(qh + (int64_t)r * 64 + (tid & 7) * 8);
    if (tid < kQT64) {
      const int rm = qt * kQT64 + tid;
      mv = rm < a.Nq ? mrow[rm] : INFINITY;   // rows past the window contribute exp2(-inf) = 0
    }
  };
  auto store_q = [&](int buf, const u32x4_t& st, float mv) {
    lq[buf][(tid >> 3) * kK64St + (tid & 7)] = st;
    if (tid < kQT64) lm[buf][tid] = mv;
  };
  u32x4_t st;
  float mv = 0.f;
  load_q(0, st, mv);
  store_q(0, st, mv);
  __syncthreads();
  const float c2 = a.scale * 1.4426950408889634f;
  const int qbase = l32 * kK64St + hl;
  float acc = 0.f;
  for (int qt = 0; qt < nqt; ++qt) {
    const bool more = qt + 1 < nqt;
    if (more) load_q(qt + 1, st, mv);
    const u32x4_t* q = lq[qt & 1];
    f32x16_t c;
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, q[qbase + ks * 2]), kf[ks], c, 0, 0, 0);
    // accumulator i is query row (i/4)*8 + hl*4 + i%4 of the tile
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const float4 mg = *reinterpret_cast<const float4*>(&lm[qt & 1][g4 * 8 + hl * 4]);
      acc += __builtin_amdgcn_exp2f(fmaf(c[g4 * 4 + 0], c2, -mg.x));
      acc += __builtin_amdgcn_exp2f(fmaf(c[g4 * 4 + 1], c2, -mg.y));
      acc += __builtin_amdgcn_exp2f(fmaf(c[g4 * 4 + 2], c2, -mg.z));
      acc += __builtin_amdgcn_exp2f(fmaf(c[g4 * 4 + 3], c2, -mg.w));
    }
    if (more) store_q((qt + 1) & 1, st, mv);
    __syncthreads();
  }
  const float tot = xhalf_sum(acc);
  if (hl == 0 && key < nk) {
    const int ncap = a.keys.cap[0] + a.keys.cap[1];
    const int p = region == 0 ? key : a.keys.cap[0] + key;
    a.part[(int64_t)h * ncap + p] = tot;
  }
}

hipError_t launch_score_mfma64(const ScoreArgs& a, const uint16_t* qbf, hipStream_t s) {
  if (a.geo.D != 64 || a.geo.esz != 2 || a.geo.DA != kD64A || a.geo.DB != kD64B) return hipErrorInvalidValue;
  const int ntile0 = range_tiles(a.keys, 0);
  const int ntile1 = range_tiles(a.keys, 1);
  ScoreArgs b = a;
  int n0 = ntile0, nt = ntile0 + ntile1;
  if (ntile0 == 0) {   // keep region 0 non-empty for the tile sequence
    b.keys.ka[0] = a.keys.ka[1];
    b.keys.kb[0] = a.keys.kb[1];
    b.keys.v[0] = a.keys.v[1];
    b.keys.t[0] = a.keys.t[1];
    b.keys.cap[0] = a.keys.cap[1];
    b.keys.lo[0] = a.keys.lo[1];
    b.keys.n[0] = a.keys.n[1];
    b.keys.lo[1] = 0;
    b.keys.n[1] = 0;
    n0 = ntile1;
    nt = ntile1;
  }
  if (nt == 0 || a.Nq == 0) return hipSuccess;
  if (!a.rows_given) {   // else a.m holds the attention's row normalisers
    const int mblocks = (a.Nq + kBM - 1) / kBM;
    const int total = mblocks * a.geo.H;
    hipLaunchKernelGGL(score_rows_d64_kernel, dim3(total), dim3(256), 0, s, b, qbf, mblocks, total, n0, nt);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  // columns: original region numbering (part is indexed by physical slot)
  for (int r = 0; r < 2; ++r) {
    if (a.keys.n[r] == 0) continue;
    const int kblocks = (a.keys.n[r] + 127) / 128;
    const int tot = kblocks * a.geo.H;
    hipLaunchKernelGGL(score_cols_d64_kernel, dim3(tot), dim3(256), 0, s, a, qbf, r, kblocks, tot);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// v5f: v5 with a fixed reference per row instead of a running maximum.  Every
// row keeps m = max of its scores in tile 0 (log2 units) for all tiles, so a
// tile needs no maximum, no rescale test and no O rescale: P = exp2(c2 s - m).
// The result is the same normalisation (a constant shift cancels between O and
// the row sum), exact up to rounding while P stays in range.  A row whose later
// scores exceed m so far that a 32-term partial sum of P passes 2^48 (or turns
// inf/NaN) marks its block in a.flags, and the running-maximum v5 kernel then
// recomputes exactly the marked blocks.
// S^T(t+1) on the matrix cores, interleaved with P(t) = exp2(c2 S^T(t) - m)
__device__ __forceinline__ void qk_and_exp(f32x16_t* s, const u32x4_t* lk, const bf16x8_t* qf, int kbase,
                                           const f32x16_t* sp, float negm, float c2, bf16x8_t pb[2][2],
                                           float& psum) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  psum = 0.f;
#pragma unroll
  for (int step = 0; step < 16; ++step) {
    const int kb = step & 1, ks = step >> 1;      // the two accumulators alternate
    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, lk[kbase + kb * 32 * kKSt + ks * 2]);
    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks], s[kb], 0, 0, 0);
    const int e = step * 2;
    const int pkb = e >> 4, phf = (e >> 3) & 1, pj = e & 7;
    const float p0 = __builtin_amdgcn_exp2f(fmaf(sp[pkb][phf * 8 + pj], c2, negm));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(sp[pkb][phf * 8 + pj + 1], c2, negm));
    const bf16x2_t pr = {(__bf16)p0, (__bf16)p1};
    pb[pkb][phf][pj] = pr[0];
    pb[pkb][phf][pj + 1] = pr[1];
    psum = __builtin_amdgcn_fdot2_f32_bf16(pr, one, psum, false);
  }
  asm volatile("" ::"v"(psum));
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) asm volatile("" ::"v"(__builtin_bit_cast(u32x4_t, pb[kb][hf])));
  __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);     // six operand reads ahead (eight spill)
#pragma unroll
  for (int step = 0; step < 16; ++step) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);
  }
}

template <bool CAUSAL>
__global__ __launch_bounds__(512, 1) void attend_v5f_kernel(AttendArgs a, int mblocks, int total, int per_xcd,
                                                           int ntile0, int ntiles, int kparts) {
  __shared__ u32x4_t lks[2][kKTileP];
  __shared__ u32x4_t lvs[2][kVTileP];
  __shared__ int s_flag;
  const int wg = blockIdx.x;
  // unit order and key parts as in the running-maximum kernel (block-causal: longest first, round-robin
  // over the XCDs; split keys: kparts balanced parts of the tile sequence, never when causal)
  const int lin = CAUSAL ? wg : (wg & 7) * per_xcd + (wg >> 3);
  if (lin >= total) return;
  const int hp = CAUSAL ? lin % a.geo.H : lin / mblocks;   // head * kparts + part
  const int h = hp / kparts, part = hp - h * kparts;
  const int mb = CAUSAL ? mblocks - 1 - lin / a.geo.H : lin - hp * mblocks;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int qrow = mb * 256 + wave * 32 + l32;
  // not causal: whole tiles first, the few edge tiles (which need masks) last
  TileSeq ts = CAUSAL ? tile_seq(a.keys, ntile0, ntiles) : tile_seq_edges_last(a.keys, ntile0, ntiles);
  ts.first = part * ntiles / kparts;
  const int kbase = perm_row(l32) * kKSt + hl;
  const int vbase = l32 * kVSt + hl;
  // block-causal limits, as in the running-maximum kernel
  int nt = (part + 1) * ntiles / kparts - ts.first, lim = 0, lim_lo = 0;
  if (CAUSAL) {
    const int cb = a.causal_block, nall = a.keys.n[0] + a.keys.n[1];
    auto limit = [&](int r) { return min(nall, (r / cb + 1) * cb); };
    const int r0 = mb * 256, r1 = min(a.Lq, r0 + 256) - 1;
    lim_lo = limit(r0);
    lim = limit(min(qrow, a.Lq - 1));
    const int lim_hi = limit(r1), n0 = a.keys.n[0];
    nt = lim_hi <= n0 ? (lim_hi + kBN - 1) / kBN : ntile0 + (lim_hi - n0 + kBN - 1) / kBN;
  }
  const int last = nt - 1;
  auto mask = [&](f32x16_t* s, int t) {
    const int nv = CAUSAL ? ts.valid_w(t) : ts.valid(t);   // causal: logical order
    if (CAUSAL) {
      const int lb = t < ntile0 ? t * kBN : a.keys.n[0] + (t - ntile0) * kBN;
      if (lb + kBN > lim_lo) {
        mask_tile_end(s, min(nv, lim - lb), hl);
        return;
      }
    }
    mask_tile(s, CAUSAL ? ts.lead_w(t) : ts.lead(t), nv, hl);
  };
  // tile lookups of the prologue (logical order when causal)
  auto reg = [&](int t) { return CAUSAL ? ts.region_w(t) : ts.region(t); };
  auto bas = [&](int t) { return CAUSAL ? ts.base_w(t) : ts.base(t); };
  const TilePtrs tp = tile_ptrs(a.keys, h, tid);
  if (tid == 0) s_flag = 0;

  Stage5 st;
  load5(st, tp, reg(0), bas(0), reg(0), bas(0));
  bf16x8_t qf[8];
  load_query(qf, a, h, min(qrow, a.Lq - 1), hl);
  store5(st, lks[0], lvs[0], tid, true, true);
  {
    const int t1 = min(1, last);
    load5(st, tp, reg(t1), bas(t1), 0, 0);
    store5(st, lks[1], lvs[1], tid, true, false);
  }
  f32x16_t o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
  float lsum = 0.f, pmax = 0.f;
  const float c2 = a.scale * 1.4426950408889634f;
  __syncthreads();
  f32x16_t sa[2], sb[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sa[kb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, lks[0][kbase + kb * 32 * kKSt + ks * 2]);
      sa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks], sa[kb], 0, 0, 0);
    }
  }
  mask(sa, 0);
  // tile 0 holds at least one valid key (for every row, also block-causal), so the reference is finite
  const float negm = -tile_max(sa, c2);
  __syncthreads();   // every wave has read K(0) before step 0 stores K(2) over it

  auto step = [&](int t, f32x16_t* scur, f32x16_t* snext, auto masked) {
    const int tk = min(t + 2, last), tv = min(t + 1, last);
    // clean steps load only tiles visited before the edges (or any tile in logical order)
    constexpr bool any = decltype(masked)::value && !CAUSAL;
    const int rk = any ? ts.region(tk) : ts.region_w(tk), bk = any ? ts.base(tk) : ts.base_w(tk);
    const int rv = any ? ts.region(tv) : ts.region_w(tv), bv = any ? ts.base(tv) : ts.base_w(tv);
    load5(st, tp, rk, bk, rv, bv);
    bf16x8_t pb[2][2];
    float psum;
    qk_and_exp(snext, lks[(t + 1) & 1], qf, kbase, scur, negm, c2, pb, psum);
    pmax = fmaxf(pmax, psum);
    lsum += psum;
    pv_padded(o, lvs[t & 1], vbase, pb);
    if constexpr (decltype(masked)::value) mask(snext, min(t + 1, last));
    store5(st, lks[t & 1], lvs[(t + 1) & 1], tid, true, true);
    __syncthreads();
  };
  using Masked = std::integral_constant<bool, true>;
  using Clean = std::integral_constant<bool, false>;

  // the leading steps whose next tile (t + 1) needs no mask run without the mask code (its branches and
  // temporaries otherwise cost the loop issue slots and registers); steps 0 .. clean - 1 are such steps.
  // Not causal: the whole tiles the edges-last order visits first.  Block-causal: the whole tiles that
  // end before every row's limit.
  int clean = CAUSAL ? 0 : max(0, ts.whole_prefix(nt) - 2);   // tile t + 2 (loaded ahead) is whole too
  if (CAUSAL) clean = causal_clean_steps(a.keys.n[0], a.keys.n[1], ntile0, nt, lim_lo);
  int t = 0;
  for (; t + 1 < clean; t += 2) {
    step(t, sa, sb, Clean{});
    step(t + 1, sb, sa, Clean{});
  }
  for (; t + 1 < nt; t += 2) {
    step(t, sa, sb, Masked{});
    step(t + 1, sb, sa, Masked{});
  }
  if (t < nt) step(t, sa, sb, Masked{});
  if (__ballot(!(pmax <= kPLimit)) != 0 && lane == 0) s_flag = 1;
  __syncthreads();
  if (tid == 0) a.flags[lin] = s_flag;
  if (kparts > 1)
    store_partial(a, o, -negm, lsum, qrow, h, part, hl);   // the fixed reference, log2 units like v5's max
  else
    store_out(a, o, lsum, qrow, h, hl, -negm);
}

// Launch shapes of the matrix-core attention.
enum class AttendPlan { kFixedRef, kRunningMax, kCausalFixedRef, kCausalRunningMax, kSplit };

// b = a with region 0 non-empty (a region with no valid keys contributes no tiles), n0 / nt = region 0's
// tiles and all tiles; false when there is no work
static bool attend_regions(const AttendArgs& a, AttendArgs& b, int& n0, int& nt) {
  const int ntile0 = range_tiles(a.keys, 0);
  const int ntile1 = range_tiles(a.keys, 1);
  b = a;
  n0 = ntile0;
  nt = ntile0 + ntile1;
  if (a.Lq == 0 || a.geo.H == 0 || nt == 0) return false;
  if (ntile0 == 0) {
    b.keys.ka[0] = a.keys.ka[1];
    b.keys.kb[0] = a.keys.kb[1];
    b.keys.v[0] = a.keys.v[1];
    b.keys.t[0] = a.keys.t[1];
    b.keys.cap[0] = a.keys.cap[1];
    b.keys.lo[0] = a.keys.lo[1];
    b.keys.n[0] = a.keys.n[1];
    b.keys.lo[1] = 0;
    b.keys.n[1] = 0;
    n0 = ntile1;
    nt = ntile1;
  }
  return true;
}

static hipError_t attend_launch(const AttendArgs& a, AttendPlan plan, hipStream_t s) {
  const int mblocks = (a.Lq + 255) / 256;
  const int total = mblocks * a.geo.H;
  const int per_xcd = (total + 7) / 8;
  AttendArgs b;
  int n0, nt;
  if (!attend_regions(a, b, n0, nt)) return hipSuccess;
  const dim3 grid(8 * per_xcd), block(512);
  switch (plan) {
    case AttendPlan::kSplit: {   // fixed-reference partials, flagged parts again, then the merge
      const int kp = split_parts(total, nt);
      const int tot = total * kp, pxcd = (tot + 7) / 8;
      hipLaunchKernelGGL((attend_v5f_kernel<false>), dim3(8 * pxcd), block, 0, s, b, mblocks, tot, pxcd, n0, nt, kp);
      if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
      hipLaunchKernelGGL((attend_v5_kernel<false>), dim3(8 * pxcd), block, 0, s, b, mblocks, tot, pxcd, n0, nt,
                         (const int32_t*)b.flags, kp);
      if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
      const int64_t threads = (int64_t)a.geo.H * a.Lq * 32;
      hipLaunchKernelGGL(merge_split_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, b, kp);
      break;
    }
    case AttendPlan::kRunningMax:
      hipLaunchKernelGGL((attend_v5_kernel<false>), grid, block, 0, s, b, mblocks, total, per_xcd, n0, nt,
                         (const int32_t*)nullptr, 1);
      break;
    case AttendPlan::kCausalRunningMax:
      hipLaunchKernelGGL((attend_v5_kernel<true>), grid, block, 0, s, b, mblocks, total, per_xcd, n0, nt,
                         (const int32_t*)nullptr, 1);
      break;
    case AttendPlan::kCausalFixedRef:   // fixed reference, then the flagged blocks with the running maximum
      hipLaunchKernelGGL((attend_v5f_kernel<true>), grid, block, 0, s, b, mblocks, total, per_xcd, n0, nt, 1);
      if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
      hipLaunchKernelGGL((attend_v5_kernel<true>), grid, block, 0, s, b, mblocks, total, per_xcd, n0, nt,
                         (const int32_t*)b.flags, 1);
      break;
    case AttendPlan::kFixedRef:
      hipLaunchKernelGGL((attend_v5f_kernel<false>), grid, block, 0, s, b, mblocks, total, per_xcd, n0, nt, 1);
      if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
      hipLaunchKernelGGL((attend_v5_kernel<false>), grid, block, 0, s, b, mblocks, total, per_xcd, n0, nt,
                         (const int32_t*)b.flags, 1);
      break;
  }
  return hipGetLastError();
}

// Default: the fixed-reference kernel plus the recompute pass (it needs the
// workspace flags; without them the running-maximum kernel runs alone); split
// keys for launches with fewer workgroups than CUs when the workspace holds
// the partials.  kPathRunningMax / kPathNoSplit select the alternatives.  Keys
// must be stored rotated (a raw-key cache's time band is placed first).
hipError_t launch_attend_mfma(const AttendArgs& a, uint32_t paths, hipStream_t s) {
  if (a.raw) return hipErrorInvalidValue;
  const bool running_max = (paths & kPathRunningMax) != 0 || a.flags == nullptr;
  if (a.split_o && a.causal_block == 0 && !(paths & kPathNoSplit) && !running_max) {
    const int total = (a.Lq + 255) / 256 * a.geo.H;
    const int kp = split_parts(total, range_tiles(a.keys, 0) + range_tiles(a.keys, 1));
    if (total < 256 && kp >= 2 && (int64_t)kp * a.geo.H * a.Lq <= kSplitRows)
      return attend_launch(a, AttendPlan::kSplit, s);
  }
  if (a.causal_block > 0)
    return attend_launch(a, running_max ? AttendPlan::kCausalRunningMax : AttendPlan::kCausalFixedRef, s);
  return attend_launch(a, running_max ? AttendPlan::kRunningMax : AttendPlan::kFixedRef, s);
}

// bf16, head_dim 64: the running-maximum kernel of that width (keys stored rotated; plain or block-causal)
hipError_t launch_attend_mfma64(const AttendArgs& a, hipStream_t s) {
  if (a.raw || a.geo.D != 64 || a.geo.esz != 2 || a.geo.DA != kD64A || a.geo.DB != kD64B)
    return hipErrorInvalidValue;
  const int mblocks = (a.Lq + 255) / 256;
  const int total = mblocks * a.geo.H;
  const int per_xcd = (total + 7) / 8;
  AttendArgs b;
  int n0, nt;
  if (!attend_regions(a, b, n0, nt)) return hipSuccess;
  if (a.causal_block > 0)
    hipLaunchKernelGGL((attend_d64_kernel<true>), dim3(8 * per_xcd), dim3(512), 0, s, b, mblocks, total, per_xcd, n0,
                       nt);
  else
    hipLaunchKernelGGL((attend_d64_kernel<false>), dim3(8 * per_xcd), dim3(512), 0, s, b, mblocks, total, per_xcd,
                       n0, nt);
  return hipGetLastError();
}

}  // namespace kvc
