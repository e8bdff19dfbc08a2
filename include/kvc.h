/*
 * kvc.h -- C ABI of libkvc: a bounded, ring-indexed KV cache for chunk-wise
 * causal video attention on AMD Instinct MI355X (gfx950).
 *
 * What the cache is (sources, by page and section):
 *  - A per-layer cache of fixed capacity allocated up front: kv_size =
 *    frame_seqlen * local_attn_size (LingBot-World 2.0 sliding-window
 *    article, "chunked inference"); memory precomputed once (rCM
 *    length-extrapolation article, introduction: cache_max_len()).
 *  - The first sink_size frames are pinned; later frames roll FIFO through
 *    the remaining window; when new + local_end > kv_size the oldest
 *    non-sink tokens are evicted (LingBot article, "how the window rolls when
 *    full" and "sink_size attention sink").  Here eviction is a ring-head
 *    advance: no cached byte moves.
 *  - New keys are rotated at their absolute frame number (LingBot article,
 *    "two easily missed details"; Causal-Forcing article, section 3).
 *  - Only the current chunk's queries are computed; they attend to the cached
 *    history plus the new chunk (Causal-Forcing article, section 3).
 *  - Cached keys can be re-timed in place (rCM article, strategy 4:
 *    rope_time_delta_; strategy 3: shift, clamp to 0, RoPE cut), compacted to
 *    a kept subset (strategy 3 KV flush, strategy 4 KVCache.compact_), scored
 *    by received attention (strategy 4), and the sink refilled from a bank
 *    of the first blocks (strategy 2; Rolling Sink summary, "method step
 *    details").
 *
 * Conventions for every call:
 *  - Device pointers are HIP device (or managed) addresses; host pointers are
 *    ordinary CPU memory.  Each parameter says which.
 *  - Tensors are dense row-major.  q, k, v and out are [tokens, heads,
 *    head_dim]; tokens are frame-major, each frame row-major over its
 *    (grid_h x grid_w) latent grid.
 *  - Element type is the cache dtype (KVC_BF16: bfloat16, KVC_F32: float).
 *  - All GPU work is enqueued on the handle's stream, asynchronously, unless
 *    stated otherwise.  Inputs must stay valid until that work completes.
 *  - Every argument is validated on the host before anything is enqueued;
 *    on any error except KVC_EDEVICE the cache state is unchanged.
 *    KVC_EDEVICE (a HIP launch/copy failure) poisons the handle: every later
 *    call returns KVC_ESTATE until kvc_destroy.
 *  - kvc_last_error() returns a thread-local description of the last error.
 *  - A handle is not thread-safe; distinct handles are independent.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvc_cache* kvc_handle;

typedef enum {
  KVC_OK = 0,
  KVC_EINVAL = 1,        /* bad argument; state unchanged                      */
  KVC_ENOMEM = 2,        /* workspace too small / host allocation failed       */
  KVC_ESTATE = 3,        /* call not valid in the current state, or poisoned   */
  KVC_EDEVICE = 4,       /* HIP runtime error; the handle is poisoned          */
  KVC_EUNSUPPORTED = 5   /* feature not reserved at creation                   */
} kvc_status;

typedef enum { KVC_BF16 = 0, KVC_F32 = 1 } kvc_dtype;

/* kvc_attend: rotate q at the newest chunk's current time index. */
#define KVC_T_NEWEST INT32_MIN
/* kvc_append: re-write the newest chunk's slots in place (a denoising step
 * before the clean commit); nothing is evicted and global indices are kept. */
#define KVC_APPEND_REPLACE_NEWEST 1u
/* kvc_create: reserve the second window buffer that kvc_compact gathers into. */
#define KVC_CREATE_COMPACT 1u
/* kvc_create: raw-key cache (the MemRoPE variant of the rCM length-extrapolation
 * article: keys kept un-rotated, placed at attention time).  Keys are stored
 * with their height and width bands rotated (those positions never change)
 * and the time band raw; kvc_attend rotates each key's time band at its slot's
 * current time, so every attended key equals a fresh rotation of the raw key
 * and kvc_retime only rewrites time indices.  For bf16 caches with head_dim
 * 128 or 64 the workspace holds a copy of the keys' time-band plane that each
 * kvc_attend first fills, in one pass, with every slot (and the memory
 * tokens) placed at its current time; the attention then reads it (other
 * caches rotate inside the attention kernel).  kvc_score and kvc_relax_scores
 * see the keys placed the same way (their scratch then also holds such a copy;
 * the *_scratch_bytes calls include it). */
#define KVC_CREATE_RAW_KEYS 2u
/* kvc_create: MemRoPE memory tokens (rCM length-extrapolation article: evicted
 * frames are compressed into long- and short-term EMA memories instead of
 * dropped); needs KVC_CREATE_RAW_KEYS.  Two memory frames (long, short), one
 * token per grid position, live in 2 * frame_seqlen extra sink-region slots.
 * Every frame a kvc_append evicts (whole frames, oldest first) updates both,
 * per position, as M = a*M + (1-a)*E over the stored keys and the values, in
 * fp32 with the products and the sum rounded separately; the first evicted
 * frame initialises them (rates: kvc_set_memory_rates, default 0.9 / 0.5).
 * Once a frame has been folded, kvc_attend also attends to the memories,
 * rounded to the cache dtype and placed just before the oldest window entry
 * (long at t_w - 2, short at t_w - 1).  kvc_compact, kvc_sink_push and
 * block-causal attention return KVC_EUNSUPPORTED on such a cache. */
#define KVC_CREATE_MEMORY 4u
/* kvc_create: reserve 65 MB of workspace for split-key attention.  When a
 * kvc_attend call would give fewer 256-query workgroups than the GPU has
 * compute units (few heads, short chunks: e.g. one GPU's share of a
 * head-sharded layer), the keys are cut into 2-8 parts that run as separate
 * workgroups, and a merge pass combines their partial results.  Without the
 * flag such calls run unsplit. */
#define KVC_CREATE_SPLIT_ATTEND 8u
/* Largest |time index| and |retime delta| (the RoPE time table covers
 * positions -KVC_MAX_POS .. KVC_MAX_POS). */
#define KVC_MAX_POS 16383
/* Largest number of query frames per kvc_attend / kvc_score call. */
#define KVC_MAX_Q_FRAMES 32

typedef struct {
  int32_t capacity;        /* (sink_frames + window_frames) * frame_seqlen        */
  int32_t n_valid;         /* valid entries = sink_filled + window_filled          */
  int32_t sink_tokens;     /* sink capacity in tokens                              */
  int32_t window_tokens;   /* rolling window capacity in tokens                    */
  int32_t sink_filled;
  int32_t window_filled;
  int32_t sink_head;       /* physical slot of the oldest sink entry               */
  int32_t window_head;     /* physical slot of the oldest window entry             */
  int64_t global_end;      /* tokens appended so far (not counting re-writes)      */
  int32_t newest_valid;    /* 1 if the newest chunk is still whole in the cache    */
  int32_t newest_frames;
  int32_t newest_t;        /* current time index of the newest chunk's first frame */
  int32_t bank_tokens;     /* raw-key bank capacity (Rolling Sink), 0 if none      */
  int64_t newest_g;        /* global index of the newest chunk's first token       */
  int32_t bank_complete;   /* 1 once global_end >= bank_tokens                     */
  int32_t window_buffer;   /* which of the two window buffers is current (0/1)     */
} kvc_info_t;

/* Device bytes the caller must provide to kvc_create for this geometry
 * (includes K/V planes, time/global-index arrays, RoPE tables, the optional
 * raw-key bank, with KVC_CREATE_COMPACT the second window buffer, with
 * KVC_CREATE_RAW_KEYS the placed time-band plane described there, and the
 * small per-block flag array kvc_attend uses to mark blocks for recompute).
 * Returns 0 for an unsupported geometry (head_dim not 64/128, bad sizes). */
size_t kvc_workspace_bytes(int32_t sink_frames, int32_t window_frames, int32_t frame_seqlen,
                           int32_t heads, int32_t head_dim, kvc_dtype dt, int32_t bank_frames,
                           uint32_t create_flags);

/* Create a cache over caller-owned device memory `workspace` (>= the size
 * above, 256-byte aligned).  grid_w is the latent grid width (frame_seqlen
 * must be a multiple of it).  The library builds the RoPE tables on the host
 * (fp64 -> fp32), zero-fills the workspace and uploads the tables on
 * `hip_stream` (hipStream_t, may be NULL for the default stream), then
 * synchronizes that stream once.  The library never allocates device memory;
 * it must not outlive `workspace`.  *out receives the handle. */
kvc_status kvc_create(int32_t sink_frames, int32_t window_frames, int32_t frame_seqlen,
                      int32_t heads, int32_t head_dim, int32_t grid_w, kvc_dtype dt,
                      int32_t bank_frames, uint32_t create_flags, void* workspace, size_t ws_bytes,
                      void* hip_stream, kvc_handle* out);

/* Layer groups: one cache per transformer layer, all over one workspace of
 * n_layers identical per-layer layouts (layer l at workspace + l *
 * kvc_workspace_bytes(...)), so that the cache operations every layer makes
 * alike between chunks -- retime, compact, sink push -- run as ONE launch over
 * the layers (the *_layers calls below).  Appends and attends stay per layer
 * (a layer's keys and queries exist only inside its own forward pass).
 * kvc_create_group fills out[0 .. n_layers-1] with handles made as by
 * kvc_create (same arguments for every layer, same stream); on failure none
 * is left created.  Each handle is destroyed with kvc_destroy. */
size_t kvc_group_workspace_bytes(int32_t n_layers, int32_t sink_frames, int32_t window_frames,
                                 int32_t frame_seqlen, int32_t heads, int32_t head_dim, kvc_dtype dt,
                                 int32_t bank_frames, uint32_t create_flags);
kvc_status kvc_create_group(int32_t n_layers, int32_t sink_frames, int32_t window_frames, int32_t frame_seqlen,
                            int32_t heads, int32_t head_dim, int32_t grid_w, kvc_dtype dt, int32_t bank_frames,
                            uint32_t create_flags, void* workspace, size_t ws_bytes, void* hip_stream,
                            kvc_handle* out);

/* Free host state; the workspace stays the caller's. */
kvc_status kvc_destroy(kvc_handle h);

/* Change the stream later calls enqueue on.  The new stream is first made to
 * wait (hipStreamWaitEvent) for the work already queued on the old one, so
 * later calls see the cache as that work leaves it; nothing else is
 * synchronized. */
kvc_status kvc_set_stream(kvc_handle h, void* hip_stream);

/* Kernel paths (bits for kvc_set_paths; 0 selects the default kernels).  They
 * exist to compare the kernels against each other and to test each one; every
 * path gives results within the attention tolerance of the others, and the
 * cache state they leave is identical.
 *  KVC_PATH_RUNNING_MAX  attention: the running-maximum kernel alone instead
 *                        of the fixed per-row reference with its recompute pass
 *  KVC_PATH_GENERAL      attention and scores: the general one-thread-per-row
 *                        passes (the only ones for fp32 caches; bf16 head_dim
 *                        64 caches otherwise run matrix-core kernels of their
 *                        own width, with a running maximum)
 *  KVC_PATH_NO_SPLIT     attention: never split the keys (KVC_CREATE_SPLIT_ATTEND) */
#define KVC_PATH_RUNNING_MAX 1u
#define KVC_PATH_GENERAL 2u
#define KVC_PATH_NO_SPLIT 4u
/* Select the kernel paths of later calls on this handle.  EINVAL for unknown
 * bits. */
kvc_status kvc_set_paths(kvc_handle h, uint32_t paths);

/* Append n_frames new frames at time indices t_index .. t_index+n_frames-1.
 * k, v: device, [n_frames*frame_seqlen, heads, head_dim] raw (un-rotated) keys
 * and values.  Keys are rotated with the 3D RoPE (time band at the absolute
 * frame, height/width bands at the token's grid position) and stored in the
 * cache dtype (bf16 round-to-nearest-even).  The first sink tokens ever
 * appended fill the sink; the rest go to the window, evicting the oldest
 * window tokens when full (ring-head advance).  While global_end <
 * bank_tokens, raw k/v are also captured into the bank.
 * flags: KVC_APPEND_REPLACE_NEWEST re-writes the newest chunk in place (its
 * frame count must match).  EINVAL if n_frames*frame_seqlen exceeds the
 * window, or |t_index|+n_frames exceeds KVC_MAX_POS.  k and v must be
 * finite for attention to be defined: attention weights the unused slots of a
 * partial key tile by exactly zero, so a non-finite value left in a slot after
 * its entry was dropped by a compaction can still reach a later attend's
 * output.  (Storage itself is defined for any input: a NaN is stored as the
 * quiet bf16 NaN 0x7FC0 with its sign, infinities as infinities.) */
kvc_status kvc_append(kvc_handle h, const void* k, const void* v, int32_t n_frames, int32_t t_index,
                      uint32_t flags);

/* out = softmax(q_hat K^T / sqrt(head_dim)) V over every valid entry (sink,
 * window and the newest chunk), with no mask.  q: device, [q_frames *
 * frame_seqlen, heads, head_dim] raw queries, rotated here at time q_t_index
 * + frame (KVC_T_NEWEST: the newest chunk's current time) and rounded to the
 * cache dtype.  out: device, same shape and dtype.  ESTATE if the cache is
 * empty.  Uses the handle's workspace flags, so attends on one handle must not
 * overlap on different streams. */
kvc_status kvc_attend(kvc_handle h, const void* q, int32_t q_frames, int32_t q_t_index, void* out);

/* Block-causal attention of a whole clip (the clip-level training /
 * teacher-forcing path: rCM length-extrapolation article, block-level
 * attention mask; Causal-Forcing article, section 4, a 21-frame clip split
 * into blocks of num_frame_per_block frames).  Query frame f (rotated at
 * q_t_index + f, as in kvc_attend) belongs to block f / block_frames and
 * attends to the first min(n_valid, (block + 1) * block_frames *
 * frame_seqlen) cached entries in logical order -- i.e. to blocks 0..its own
 * when the cache holds the clip from its first frame.  q, out as in
 * kvc_attend.  EINVAL for block_frames outside 1..KVC_MAX_Q_FRAMES;
 * EUNSUPPORTED once the window ring has wrapped or the sink rolled (logical
 * order no longer equals slot order); ESTATE if the cache is empty. */
kvc_status kvc_attend_blockcausal(kvc_handle h, const void* q, int32_t q_frames, int32_t q_t_index,
                                  int32_t block_frames, void* out);

/* Shift the time index of logical entries [slot_lo, slot_hi) by delta
 * (clamped at 0 when clamp0 != 0) and re-rotate their stored keys' time band
 * in place by the actual change.  Logical order: sink oldest..newest, then
 * window oldest..newest.  EINVAL if the range is outside [0, n_valid) or a
 * resulting |time| exceeds KVC_MAX_POS. */
kvc_status kvc_retime(kvc_handle h, int32_t delta, int32_t clamp0, int32_t slot_lo, int32_t slot_hi);

/* kvc_retime / kvc_compact / kvc_sink_push over n_layers layers in one launch:
 * layers[0 .. n_layers-1] must be consecutive members of one kvc_create_group
 * group (layer index increasing by one), on the same stream and in the same
 * cache state (as they are when every layer received the same calls); EINVAL
 * otherwise, ESTATE if the states differ.  The result on every layer is what
 * the single-layer call would give.  A HIP failure poisons all of them. */
kvc_status kvc_retime_layers(const kvc_handle* layers, int32_t n_layers, int32_t delta, int32_t clamp0,
                             int32_t slot_lo, int32_t slot_hi);
kvc_status kvc_compact_layers(const kvc_handle* layers, int32_t n_layers, const int32_t* keep_idx, int32_t n_keep);
kvc_status kvc_sink_push_layers(const kvc_handle* layers, int32_t n_layers, int32_t bank_frame, int32_t n_frames,
                                int32_t t_index);

/* Device scratch bytes kvc_score needs for q_frames query frames. */
size_t kvc_score_scratch_bytes(kvc_handle h, int32_t q_frames);

/* Attention mass received by each valid entry from a window of queries,
 * summed over heads and query rows: scores[j] = sum_h sum_i softmax_j(q_hat_i
 * . k_j / sqrt(head_dim)).  q_win: device [q_frames*frame_seqlen, heads,
 * head_dim] raw queries; q_t: host int32[q_frames], the time index of each
 * query frame (copied before return); scores: device float[n_valid] in
 * logical order; scratch: device, >= kvc_score_scratch_bytes. */
kvc_status kvc_score(kvc_handle h, const void* q_win, int32_t q_frames, const int32_t* q_t, float* scores,
                     void* scratch, size_t scratch_bytes);

/* Attention that also keeps each query row's softmax normaliser, so that a
 * later score of the same queries over the same entries needs only its
 * columns pass.  Deep Forcing (rCM length-extrapolation article, strategy 4)
 * scores the entries by the attention the previous chunk's queries paid to
 * them, and nothing changes the cache between that attention and the scoring.
 * As kvc_attend, plus row_stats: device float[heads][q_frames *
 * frame_seqlen], caller-owned; row_stats[h][i] = log2 sum_j exp2(c * q_hat_i .
 * k_j) over the valid entries, c = log2(e) / sqrt(head_dim).  EINVAL if
 * row_stats is NULL; EUNSUPPORTED when the attention would read other entries
 * than a score does (a KVC_CREATE_MEMORY cache after its first fold, or an
 * attention limit below the number of entries).  The handle remembers the
 * latest such call (buffer, frames, times) until the next call that changes
 * the entries. */
kvc_status kvc_attend_stats(kvc_handle h, const void* q, int32_t q_frames, int32_t q_t_index, void* out,
                            float* row_stats);

/* kvc_score with the rows pass replaced by row_stats from kvc_attend_stats:
 * the same scores (up to rounding: the attention sums its probabilities as
 * rounded to the cache dtype) at about half the work.  row_stats must be the
 * buffer of the handle's latest kvc_attend_stats, made with the same query
 * frames (q_t[f] = its time + f) over the current entries: no append, retime,
 * compact, sink push or attention-limit change since (KVC_ESTATE otherwise).
 * The query window q_win must hold the same queries; that is the caller's to
 * keep.  Other arguments and errors as kvc_score. */
kvc_status kvc_score_with_stats(kvc_handle h, const void* q_win, int32_t q_frames, const int32_t* q_t,
                                const float* row_stats, float* scores, void* scratch, size_t scratch_bytes);

/* Limit what kvc_attend reads to the newest max_keys valid entries in logical
 * order (LingBot-World 2.0 article, max_attention_size: queries read only the
 * last max_attention_size positions of the cache buffer, sink first), i.e. the
 * oldest entries -- the sink first once the limit is below the window's
 * length -- drop out of attention without leaving the cache.  0 (the default)
 * = no limit.  EINVAL if max_keys < 0.  A limited attend (max_keys below the
 * number of entries) returns KVC_EUNSUPPORTED when the visible entries span a
 * Rolling-Sink sink that has rolled, on a KVC_CREATE_MEMORY cache (before its
 * first fold too), or for block-causal attention. */
kvc_status kvc_set_attention_limit(kvc_handle h, int32_t max_keys);

/* Memory-token rates (KVC_CREATE_MEMORY caches): alpha_long for the long
 * memory, alpha_short for the short one, each in [0, 1]; they apply to the
 * frames folded from the next eviction on.  EUNSUPPORTED without memory. */
kvc_status kvc_set_memory_rates(kvc_handle h, float alpha_long, float alpha_short);

/* Copy the memory tokens out (for inspection; synchronizes the stream):
 * k, v: device, [2 * frame_seqlen, heads, head_dim] in the cache dtype, the
 * long memory's tokens then the short one's, keys in stored form (height and
 * width bands rotated, time band raw); *n_folded (host) = frames folded so far
 * (0: the memories are empty and not attended).  EUNSUPPORTED without memory. */
kvc_status kvc_export_memory(kvc_handle h, void* k, void* v, int32_t* n_folded);

/* Device scratch bytes kvc_relax_scores needs (depends only on the cache
 * geometry). */
size_t kvc_relax_scratch_bytes(kvc_handle h);

/* Relax Forcing frame scores (rCM length-extrapolation article, strategy 5:
 * the cache is Sink + History + Tail; History frames are ranked by
 * score = weight * alignment + (1 - weight) * complement and the Top-K kept).
 * The cache must hold whole frames: frame f is logical entries [f * S,
 * (f + 1) * S).  The Tail is the last tail_frames frames; the candidates are
 * the n_cand = n_valid / S - sink_filled / S - tail_frames frames between the
 * sink and the Tail.  With x_f the sum of frame f's stored keys over its
 * tokens (flattened over heads and dims) and x_T the sum over the Tail's:
 *   alignment(f)  = cos(x_f, x_T)
 *   complement(f) = 1 - mean over the other candidates g of cos(x_f, x_g)
 *                   (1 when f is the only candidate)
 * with cos = 0 when either vector is zero.  scores: device float[n_cand], in
 * candidate order; scratch: device, 256-byte aligned, >=
 * kvc_relax_scratch_bytes.  EINVAL if a frame is partial, tail_frames < 1,
 * no candidate is left, weight is outside [0, 1] or a pointer is null;
 * ENOMEM if the scratch is too small; EUNSUPPORTED for more than 64 frames
 * (candidates + Tail) in one call.  The cache state is not changed. */
kvc_status kvc_relax_scores(kvc_handle h, int32_t tail_frames, float weight, float* scores, void* scratch,
                            size_t scratch_bytes);

/* Bytes of the scratch the library holds for kvc_relax_scores_noalloc, per GPU. */
#define KVC_RELAX_NOALLOC_SCRATCH_BYTES (8u << 20)
/* kvc_relax_scores for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops that forbid allocation): the same
 * computation and result, with the scratch taken from an array of
 * KVC_RELAX_NOALLOC_SCRATCH_BYTES that the library holds in each GPU's memory
 * from the first such call on that GPU until the process ends.  Allocates
 * nothing.  ENOMEM, before anything is enqueued, when the cache needs more
 * scratch than that (kvc_relax_scratch_bytes(h) > KVC_RELAX_NOALLOC_SCRATCH_BYTES);
 * other errors as kvc_relax_scores.  Every call on one GPU uses the same array
 * and nothing in it needs to start at zero (a call writes every element it
 * reads): calls ordered on one stream are safe, calls that overlap in time on
 * one GPU (other streams, other host threads) race. */
kvc_status kvc_relax_scores_noalloc(kvc_handle h, int32_t tail_frames, float weight, float* scores);

/* Keep exactly the logical entries keep_idx[0..n_keep) (host int32, sorted,
 * unique, in [0, n_valid), containing every sink entry), packed in that
 * order; window entries are gathered into the other window buffer.  Requires
 * KVC_CREATE_COMPACT (else EUNSUPPORTED).  The newest chunk stays
 * addressable for REPLACE_NEWEST only if all of it is kept. */
kvc_status kvc_compact(kvc_handle h, const int32_t* keep_idx, int32_t n_keep);

/* Rolling-Sink sink step: drop the oldest n_frames sink frames and append
 * bank frames [bank_frame, bank_frame+n_frames) (raw keys captured during the
 * first appends), rotated afresh at times t_index .. t_index+n_frames-1.
 * ESTATE unless the bank is complete and the sink full. */
kvc_status kvc_sink_push(kvc_handle h, int32_t bank_frame, int32_t n_frames, int32_t t_index);

/* Counters (host-side, no synchronization). */
kvc_status kvc_info(kvc_handle h, kvc_info_t* out);

/* Host mirror of each valid entry's time and global index, logical order
 * (host arrays of n_valid elements; either may be NULL).  No synchronization. */
kvc_status kvc_slot_times(kvc_handle h, int32_t* t, int64_t* g);

/* Gather the valid entries in logical order: k, v device [n_valid, heads,
 * head_dim] (stored, i.e. rotated, keys), t device int32[n_valid], g device
 * int64[n_valid].  Synchronizes the stream before returning. */
kvc_status kvc_export(kvc_handle h, void* k, void* v, int32_t* t, int64_t* g);

/* Copy RoPE table rows to the host: band 0 = time (positions may be
 * negative), 1 = height, 2 = width; positions [pos_lo, pos_lo + n_pos);
 * out: host float[n_pos][band_width/2][2] as (cos, sin).  Synchronizes. */
kvc_status kvc_export_tables(kvc_handle h, int32_t band, int32_t pos_lo, int32_t n_pos, float* out);

/* Thread-local message for the last failing call on this thread. */
const char* kvc_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* KVC_H */
