// kvc_device.hpp -- argument blocks shared by the host layer and the HIP kernels.
//
// HBM layout of one cache (all per layer, head-major):
//   region r in {sink, window0, window1}: capacity cap (a multiple of 64 slots)
//     KA[H][cap][DA]   stored keys, dims [0, DA): the time band (+ padding dims
//                      of the height band so rows are 16-byte multiples);
//                      retime touches only this plane, so its traffic is
//                      dense and coalesced
//     KB[H][cap][DB]   stored keys, dims [DA, D)
//     V [H][cap/64][D][64]  values in 64-slot tiles stored transposed
//                      (d-major inside a tile): attention reads a tile as one
//                      contiguous 16 KB block already in the layout its
//                      P.V matrix-core product wants
//     t [cap] int32, g [cap] int64
//   bank (Rolling Sink): raw K, V [H][bank_tok][D]
//   RoPE tables (fp32 cos/sin pairs): time [2*MAXPOS+1][Pt][2],
//     height [grid_h][Pb][2], width [grid_w][Pb][2]
#pragma once

#include <cstdint>

namespace kvc {

constexpr int kTile = 64;        // slots per V tile / attention key tile
constexpr int kMaxSegs = 4;
// slots per retime workgroup: 8 with 24 or more heads; with fewer, 32 (16 where the time band has more
// than 8 chunks of 16 bytes), so that a workgroup still moves about as many bytes
constexpr int retime_band_chunks(int D, int esz) { return (D - 4 * (D / 6) + 16 / esz - 1) / (16 / esz); }
constexpr int retime_slots(int heads, int D, int esz) {
  return heads >= 24 ? 8 : (32 * retime_band_chunks(D, esz) <= 256 ? 32 : 16);
}

// Kernel-path bits (kvc_set_paths): alternatives to the default kernels, for
// comparisons and tests.
constexpr uint32_t kPathRunningMax = 1u;  // attention: the running-maximum kernel alone
constexpr uint32_t kPathGeneral = 2u;     // attention and scores: the general per-row passes
constexpr uint32_t kPathNoSplit = 4u;     // attention: never split keys

struct RegionPtrs {
  void* ka;
  void* kb;
  void* v;
  int32_t* t;
  int64_t* g;
  int32_t cap;
};

struct Geo {
  int32_t H, D, S, grid_w;
  int32_t DA, DB;      // plane widths
  int32_t dt, bw;      // time band width, height/width band width
  int32_t esz;         // element bytes (2 bf16, 4 f32)
};

struct Tables {
  const float* tcs;    // [(pos + maxpos)][dt/2][2]
  const float* hcs;    // [h][bw/2][2]
  const float* wcs;    // [w][bw/2][2]
  int32_t maxpos;
};

struct SegW {
  int32_t region, dst, src, n;
  int32_t kb0, vb0;    // first K-part / V-part block of this segment
};

// Layer batching: a launch with gridDim.y = L works on L caches whose
// workspaces sit layer_stride bytes apart (identical layouts); every pointer
// into a workspace is layer 0's, offset by blockIdx.y * layer_stride.
struct AppendArgs {
  int32_t layers;                         // gridDim.y (0 or 1: one layer)
  int64_t layer_stride;                   // bytes between the layers' workspaces (0: one layer)
  int64_t src_stride;                     // bytes between the layers' sources (the bank: layer_stride)
  int32_t time_raw;                       // raw-key cache: the time band is stored un-rotated
  const void* k;
  const void* v;
  int64_t k_tok, k_head, v_tok, v_head;   // element strides of the sources
  RegionPtrs reg[2];                      // [sink, current window]
  SegW seg[kMaxSegs];
  int32_t nseg;
  int32_t nkb, nvb;                       // K-part / V-part blocks
  int32_t t0;                             // time of source frame 0
  int64_t g0;                             // global index of source token 0
  void* bank_k;
  void* bank_v;
  int32_t bank_tok;
  int32_t bank_lo, bank_hi;               // source tokens captured raw into the bank at g0 + src
  Geo geo;
  Tables tab;
};

struct RangeW {
  int32_t region, lo, n;
  int32_t blk0;                           // first block of this range
  int32_t fixed, tfix;                    // placed mode: fixed != 0 places every slot at time tfix
};

struct RetimeArgs {
  int32_t layers;
  int64_t layer_stride;
  RegionPtrs reg[2];
  RangeW rng[4];
  int32_t nrng;
  int32_t delta, clamp0;
  int32_t keys;                           // 0: raw-key cache, only t changes
  void* out_ka[2];                        // non-null: rotate the stored time band by each slot's own t
                                          // (a raw-key cache placed at its times) into these KA planes
                                          // (same layout), leaving the cache and t untouched
  Geo geo;
  Tables tab;
};

struct CompactArgs {
  int32_t layers;
  int64_t layer_stride;
  RegionPtrs src, dst;
  const int32_t* idx;                     // source slot of each destination slot
  int32_t n;
  int64_t nk, nv, nt;                     // block counts, set by the launcher
  Geo geo;
};

struct ExportArgs {
  RegionPtrs reg[2];
  int32_t ns, hs, S_tok, nw, hw, W_tok;
  void* k;
  void* v;
  int32_t* t;
  int64_t* g;
  Geo geo;
};

struct KeyRegions {
  const void* ka[2];
  const void* kb[2];
  const void* v[2];
  const int32_t* t[2];                    // time index of every slot
  int32_t cap[2];
  int32_t lo[2];                          // visible slots of region r: [lo[r], n[r]) (lo is 0 unless
  int32_t n[2];                           // attention is limited to the newest entries)
};

struct AttendArgs {
  const void* q;
  void* out;
  int32_t Lq;
  int32_t t0;                             // time of query frame 0
  KeyRegions keys;
  Geo geo;
  Tables tab;
  float scale;                            // 1/sqrt(D)
  int32_t* flags;                         // workspace: one recompute flag per 256-query attention block
  int32_t causal_block;                   // > 0: query row r sees the logical key prefix min(n, (r/cb+1)*cb)
  int32_t raw;                            // raw-key cache: rotate each key's time band at its slot's t
  int32_t mem_lo;                         // region-0 slots [mem_lo, mem_lo + 2S): memory tokens ...
  int32_t mem_t[2];                       // ... placed at times mem_t[0] (first S) and mem_t[1] (next S)
  float* split_o;                         // workspace (KVC_CREATE_SPLIT_ATTEND): per key part, head and row,
  float* split_ml;                        // the unnormalised O [128] and (reference, row sum); else null
  float* row_m;                           // optional out [H][Lq]: each row's softmax normaliser in log2 units,
                                          // M = log2 sum_j exp2(c2 s_j) with c2 = log2(e)/sqrt(D), s_j = q.k_j
};

constexpr int kSplitRows = 512 * 256;     // part x head x query rows the split-key buffers hold

struct ScoreArgs {
  const void* q;                          // raw query window [Nq][H][D]
  float* qh;                              // scratch: rotated queries [H][Nq][D] (fp32 holding cache-dtype values)
  float* m;                               // scratch: row max [H][Nq]
  float* l;                               // scratch: row sum [H][Nq]
  float* part;                            // scratch: per-head column sums [H][cap0 + cap1]
  int32_t* flags;                         // scratch: one recompute flag per 256-query rows-pass block
  float* scores;                          // out: [n_valid] logical order
  int32_t rows_given;                     // 1: m already holds each row's log2 normaliser (attention row
                                          // statistics), so the rows passes are skipped
  int32_t Nq;
  int32_t qt[32];                         // time of each query frame
  KeyRegions keys;
  int32_t ns, hs, S_tok, nw, hw, W_tok;   // physical -> logical map
  Geo geo;
  Tables tab;
  float scale;
};

// MemRoPE memory tokens: fold the oldest n_frames window frames (about to be
// evicted) into the long (m = 0) and short (m = 1) EMA memories.
struct MemFoldArgs {
  RegionPtrs win;                         // the window region holding the evicted frames
  RegionPtrs sink;                        // memory slots: sink region slots [mem_lo, mem_lo + 2S)
  float* state_k;                         // [2][H][S][D] fp32
  float* state_v;                         // [2][H][D][S] fp32
  int32_t hw, W_tok;                      // window ring head and size (logical -> physical)
  int32_t n_frames;                       // frames folded, oldest first
  int32_t init;                           // 1: the first frame initialises both memories
  int32_t mem_lo;
  float alpha[2];
  Geo geo;
};

struct MemExportArgs {
  RegionPtrs sink;
  int32_t mem_lo;
  void* k;                                // [2S][H][D] stored-form keys (long, then short)
  void* v;
  Geo geo;
};

struct RelaxArgs {
  KeyRegions keys;                        // ka / kb / cap of the sink and current window
  int32_t ns, hs, S_tok, nw, hw, W_tok;   // logical -> physical map
  int32_t first;                          // logical frame of candidate 0
  int32_t n_cand, n_tail;                 // candidates, then the Tail frames right after them
  int32_t nsl;                            // token slices per frame
  float* part;                            // scratch: key sums [n_cand + n_tail][nsl][H * D]
  float* xsum;                            // scratch: frame key sums [n_cand + n_tail][H * D]
  float* gram;                            // scratch: [n_cand + n_tail]^2, upper triangle <x_i, x_j>
  float* scores;                          // out: [n_cand]
  float weight;
  Geo geo;
};

constexpr int kRelaxSlice = 256;          // tokens per frame-sum workgroup
constexpr size_t kRelaxNoallocScratch = (size_t)8 << 20;   // bytes of the library-held relax scratch per GPU
constexpr int kRelaxMaxFrames = 64;       // candidates + Tail frames per relax call (Gram matrix in LDS)

}  // namespace kvc
