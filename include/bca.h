/*
 * bca.h — block-causal chunk attention over a ring-buffer KV cache (MI355X / gfx950).
 *
 * What is computed (sources are the web pages this library is built from):
 *   - "WanToFight: Real-Time Generative Game Engine for Multi-Player Combat
 *     Interaction" (xllm-io paper review), section 3 "model components" table,
 *     rows Block-Causal Attention and Rolling KV Cache, and training Stage 2
 *     (causal adaptation): tokens attend bidirectionally inside their own chunk
 *     and, across chunks, only to the current chunk and the previous W chunks
 *     (W = 2 there); the KV of recent chunks is kept in a rolling cache that is
 *     updated after each chunk.
 *   - "Matrix-Game 4.0: Harnessing Video Models for Real-Time Playable Game
 *     Worlds" (paper summary), prerequisites "causal autoregression and KV cache"
 *     and "technical novelty": the cache keeps a recent window (20 chunks) plus a
 *     reference frame; a ring buffer overwrites the oldest slot in place instead
 *     of moving the window; the window is cut into intervals computed in
 *     parallel whose partial outputs are merged by log-sum-exp; K/V may be held
 *     in 8-bit floating point.
 *
 * For one query chunk t of one layer and one head h the result is
 *     O[i] = sum_j softmax_j(scale * <q_i, k_j>) v_j,   LSE[i] = ln sum_j exp(scale * <q_i, k_j>)
 * where j runs over exactly the keys of the visible chunks:
 *     the current chunk (k_cur, v_cur),
 *     every ring chunk c with  t - W <= c <= t - 1,
 *     the reference chunk, if use_ref is set and one has been appended.
 * Segments (num_segments) only change the order of summation: each segment is an
 * attention over a subset of keys, and the partial results are merged as
 *     M = max_g LSE_g,  w_g = exp(LSE_g - M),  O = sum_g w_g O_g / sum_g w_g,
 *     LSE = M + ln sum_g w_g.
 *
 * Conventions used by every entry point
 *   - All device buffers are owned by the caller and allocated by the caller;
 *     the library allocates no device memory and never synchronises a stream.
 *   - Dense row-major layouts:
 *       q, k_cur, v_cur, k, v, o : [n][H][d] in the stated dtype (the natural
 *                                  output of a [n, H*d] projection)
 *       lse                      : fp32 [H][n], natural logarithm
 *       cache memory             : [L][K|V][H][S+R][n][d] in kv_dtype, R = has_ref;
 *                                  the reference chunk is physical block S.
 *   - Supported (qkv dtype, kv dtype) pairs: (F32, F32), (BF16, BF16),
 *     (BF16, FP8_E4M3), (BF16, FP8_E4M3_BLOCK), (BF16, INT8K_FP8V_BLOCK).
 *     head_dim must be 64 or 128 (8-bit caches: 128, at most 64 heads).
 *   - Every argument is validated on the host before anything is enqueued. On
 *     an error nothing is enqueued and the cache state is unchanged; the return
 *     value says which class of error, bca_last_error() gives the text.
 *   - One host thread and one stream per cache. Calls are asynchronous: results
 *     are valid when the stream reaches them. The host-side slot table is
 *     updated at call time, in stream order.
 *   - No C++ exception crosses this interface.
 */
#ifndef BCA_H
#define BCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A HIP stream. This is the same type as hipStream_t; NULL is the null stream. */
struct ihipStream_t;
typedef struct ihipStream_t* bca_stream_t;

typedef enum {
  BCA_OK = 0,
  BCA_ERR_INVALID_ARG = -1,  /* bad pointer, size, index or descriptor field          */
  BCA_ERR_OUT_OF_ORDER = -2, /* chunk id went backwards, or the window is no longer
                                resident in the ring                                   */
  BCA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required            */
  BCA_ERR_UNSUPPORTED = -4,  /* dtype pair or head_dim this build has no kernel for   */
  BCA_ERR_HIP = -5           /* a HIP runtime call (launch, copy) failed              */
} bca_status;

/* BCA_FP8_E4M3_BLOCK: e4m3 codes with one scale per (layer, block, head),
 * taken from each appended chunk itself (its largest magnitude per head over
 * 448), so an append re-quantises only the block it writes ("Matrix-Game 4.0"
 * summary, technical novelty: 8-bit K/V per interval, only the changed
 * interval re-quantised). The scales live in the cache memory after the
 * blocks.
 * BCA_INT8K_FP8V_BLOCK: the same per-block scheme with K held as INT8 and V as
 * e4m3 (the same summary: each interval caches INT8 K and FP8 V). K codes are
 * symmetric int8, round to nearest even of fp32(x / scale) clamped to
 * [-127, 127] (NaN -> 0), with the block's K scale = its largest magnitude per
 * head over 127; V as in FP8_E4M3_BLOCK (over 448). Layout and scale table as
 * FP8_E4M3_BLOCK. Attention quantises each query row to two int8 terms
 * (about 15 significant bits) and takes Q K^T on the int8 matrix cores with
 * int32 accumulation, one int-to-float conversion per score; P V stays on the
 * fp8 matrix cores. */
typedef enum {
  BCA_F32 = 0,
  BCA_BF16 = 1,
  BCA_FP8_E4M3 = 2,
  BCA_FP8_E4M3_BLOCK = 3,
  BCA_INT8K_FP8V_BLOCK = 4
} bca_dtype;

typedef struct bca_cache bca_cache; /* opaque host handle */

typedef struct {
  int32_t num_layers;   /* L >= 1                                               */
  int32_t num_heads;    /* H >= 1 (8-bit caches: H <= 64)                       */
  int32_t head_dim;     /* d in {64, 128}                                       */
  int32_t chunk_tokens; /* n >= 1: tokens per chunk (query chunk = cached chunk) */
  int32_t ring_slots;   /* S in [1, 62]                                         */
  int32_t has_ref;      /* R in {0, 1}: reserve one pinned reference block       */
  int32_t kv_dtype;     /* bca_dtype of the cache: F32, BF16, FP8_E4M3,
                           FP8_E4M3_BLOCK or INT8K_FP8V_BLOCK                     */
} bca_cache_desc;

typedef struct {
  int64_t q_chunk_id;   /* t >= 0: id of the query chunk                           */
  int32_t history;      /* W in [0, S]: previous chunks visible (t-W .. t-1)       */
  int32_t use_ref;      /* 1: the reference chunk is visible if it was appended    */
  int32_t num_segments; /* G >= 1: split the visible keys into G contiguous
                           segments per query tile and merge by log-sum-exp;
                           0: the library chooses the split (balanced over the
                           device's compute units); at most 64                    */
  float scale;          /* softmax scale (finite), usually 1/sqrt(d)              */
} bca_window_spec;

/* Bytes of device memory a cache with this descriptor needs (K/V blocks of all
 * layers): per layer S ring slots plus the pinned reference block, the
 * fixed-size rolling cache of the Matrix-Game 4.0 summary (prerequisite
 * "causal autoregression and KV cache": a ring buffer of the recent window
 * and a reference frame) and of the WanToFight review (rolling KV cache of
 * the previous chunks). Returns 0 for an invalid descriptor, including one whose blocks of
 * one head ((S+R)*n*d elements) or whose chunk rows (n*H*d elements of q, k,
 * v or o) would reach 2 GiB: the kernels address those with 32-bit byte
 * offsets. */
size_t bca_cache_bytes(const bca_cache_desc* desc);

/* Creates the host handle over caller memory dev_mem (at least
 * bca_cache_bytes(desc) bytes, 256-byte aligned). All slots start empty
 * (chunk id -1) and no reference chunk is present, as at the start of a
 * rollout before the first chunk is committed (same passages as
 * bca_cache_bytes). Device memory is not touched. *out receives the handle. */
bca_status bca_cache_create(const bca_cache_desc* desc, void* dev_mem, size_t bytes,
                            bca_cache** out);

/* Frees the host handle only; the device memory stays the caller's. NULL is a
 * no-op. (Library housekeeping; the pages describe no counterpart.) */
bca_status bca_cache_destroy(bca_cache* cache);

/* FP8_E4M3 caches only. Sets the per-head dequantisation scales of one layer:
 * a stored code c means value decode(c) * scale. k_scale and v_scale are host
 * arrays of H positive finite floats, copied before return. Appends quantise
 * with round(x / scale) (fp32 division, round to nearest even, saturated to
 * +-448). Setting scales empties that layer's slots and reference block, since
 * chunks already stored were quantised with the old scales. Scales default to
 * 1.0. Matrix-Game 4.0 summary, "technical novelty" and prerequisite
 * "FP8 quantisation and CUDA Graph": attention K/V held in 8 bits. */
bca_status bca_cache_set_kv_scales(bca_cache* cache, int32_t layer, const float* k_scale,
                                   const float* v_scale);

/* Writes one chunk's K and V (device, [n][H][d] in in_dtype) into the cache in
 * place, as one fused kernel on `stream`: into ring slot chunk_id mod S, or into
 * the reference block when is_ref is 1. The slot's previous content (the oldest
 * chunk) is overwritten; nothing else moves (Matrix-Game 4.0 summary,
 * prerequisite "causal autoregression and KV cache"; WanToFight review, rolling
 * KV cache, updated after each chunk).
 * in_dtype: F32 for an F32 cache, BF16 for BF16 and FP8_E4M3 caches (quantised
 * on the fly with the layer's scales) and for FP8_E4M3_BLOCK and
 * INT8K_FP8V_BLOCK caches (the block's per-head scales are first taken from
 * this chunk, then it is quantised with them).
 * Ordering: per layer, ring chunk ids are non-decreasing; an id equal to the
 * last one re-writes that chunk in place; a smaller id returns
 * BCA_ERR_OUT_OF_ORDER. chunk_id >= 0. For is_ref the id is recorded only. */
bca_status bca_append_chunk(bca_cache* cache, int32_t layer, int64_t chunk_id, int32_t is_ref,
                            const void* k, const void* v, int32_t in_dtype, bca_stream_t stream);

/* Workspace bytes bca_attend needs for this spec (0 when it needs none): the
 * partial outputs of the window's segments before their log-sum-exp merge
 * (Matrix-Game 4.0 summary, technical novelty: the window is cut into
 * intervals computed in parallel and merged by log-sum-exp), and on 8-bit
 * caches the quantised copy of the current chunk. The figure covers any ring
 * occupancy, so one buffer sized once serves every call
 * with the same spec fields. Returns 0 as well for an invalid spec; check
 * bca_attend's status. */
size_t bca_attend_workspace_bytes(const bca_cache* cache, const bca_window_spec* spec);

/* Block-causal attention of query chunk spec->q_chunk_id of one layer.
 * q, k_cur, v_cur: device [n][H][d] in qkv_dtype; the current chunk's own K/V
 * are passed here and are never read from the ring (the chunk is committed with
 * bca_append_chunk after it is denoised: WanToFight review, section 5 "code
 * analysis"; Matrix-Game 4.0 summary, method step 4). A ring slot holding id t
 * itself is therefore not visible.
 * o: device [n][H][d] in qkv_dtype. lse: device fp32 [H][n], may be NULL.
 * workspace: device, at least bca_attend_workspace_bytes(); may be NULL when
 * that is 0. It holds the partial outputs of a split window (normalised O in
 * bf16 on a BF16 cache, fp32 otherwise, and fp32 LSE) and, on an
 * FP8_E4M3 cache, the e4m3 copy of the current chunk's K and V ([H][n][d] each,
 * quantised with the layer's per-head scales, so the chunk attends to itself
 * through the same codec as the cached chunks); an FP8_E4M3 cache always
 * needs one. Its content between calls is irrelevant; calls in flight at the
 * same time need separate workspaces.
 * FP8_E4M3 cache: both products run on the fp8 matrix cores with K and V as
 * stored; Q (scaled per query row) and the softmax weights P are each written
 * as two e4m3 terms (value and rounding residual), which keeps the result
 * within 5e-2 of attention over the stored K/V on data with 8-sigma outliers.
 * The K scale and the row's Q scale fold into the softmax scale, the V scale
 * into the output normalisation. FP8_E4M3_BLOCK: the current chunk is
 * quantised with its own per-head scales, every visible block is padded to
 * whole 64-key tiles so that each tile has one block's scales, and the
 * workspace also holds the chunk's scales ([K|V][H] fp32). INT8K_FP8V_BLOCK:
 * as FP8_E4M3_BLOCK, with the chunk's K copy in int8 and Q K^T on the int8
 * matrix cores (Q as two int8 terms per row: hi = rne(x / s), lo =
 * rne(256 (x / s - hi)), s = the row's largest magnitude over 127).
 * Errors: BCA_ERR_OUT_OF_ORDER when a chunk of the window may already have been
 * overwritten (the layer's newest ring id >= t - W + S).
 * The visible set is resolved on the host from the slot table's chunk ids each
 * call; invisible slots are never read, so their content (even NaN) cannot
 * affect the result. */
bca_status bca_attend(const bca_cache* cache, int32_t layer, const bca_window_spec* spec,
                      const void* q, const void* k_cur, const void* v_cur, int32_t qkv_dtype,
                      void* o, float* lse, void* workspace, size_t workspace_bytes,
                      bca_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * bca_attend without a workspace argument. What the workspace holds (the
 * partial outputs of a split window; on an FP8_E4M3 cache the e4m3 copy of the
 * current chunk, and its scales on an FP8_E4M3_BLOCK cache) goes to scratch
 * memory the library owns: one array of BCA_NOALLOC_SCRATCH_BYTES bytes per
 * GPU, set up on the first call on that GPU and held until the process ends.
 * The call allocates nothing. Every call on one GPU uses the same scratch
 * (nothing in it needs to start at zero, and its content after a call is
 * irrelevant), so calls that may run at the same time on one GPU (on
 * different streams, or on one stream from different host threads without
 * ordering) race and must not overlap. Arguments, results and errors as for
 * bca_attend, plus BCA_ERR_WORKSPACE when the call would need more scratch
 * than BCA_NOALLOC_SCRATCH_BYTES (the Wan- and Matrix-Game-shaped calls need
 * under 32 MiB), and BCA_ERR_HIP when the scratch address cannot be looked
 * up. */
#define BCA_NOALLOC_SCRATCH_BYTES (64u << 20)

bca_status bca_attend_noalloc(const bca_cache* cache, int32_t layer, const bca_window_spec* spec,
                              const void* q, const void* k_cur, const void* v_cur,
                              int32_t qkv_dtype, void* o, float* lse, bca_stream_t stream);

/* Rotary position embedding (RoPE) fused into the path. The pages name the step
 * only ("Matrix-Game 4.0" summary, experimental results: a RoPE fusion kernel;
 * "WorldPlay2" summary, inference optimisations: QKRoPE); the form used is the
 * common one-dimensional rotary embedding with interleaved pairs: the token at
 * position p turns each pair of dimensions (2i, 2i+1), i = 0 .. d/2-1, by the
 * angle p * rope_base^(-2i/d):
 *     (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos),
 * the same for every head. Angles are formed and reduced modulo pi/2 in double
 * precision, their cosines and sines taken in fp32 from the reduced angle, the
 * rotation done in fp32, and the result rounded to the destination
 * dtype (8-bit caches: rotated, then quantised; on a per-block cache the
 * block's K scale is taken over the rotated rows). rope_base must be finite
 * and > 0 (10000 is usual); positions must be >= 0. Token r of a chunk sits at
 * position pos0 + r; with pos0 = chunk id * n for every chunk, queries and keys
 * share one position axis and q.k depends only on the distance between tokens.
 *
 * bca_append_chunk_rope: bca_append_chunk with K rotated on its way into the
 * cache (V is stored as given). Same arguments, ordering and errors, plus
 * rope_base and pos0.
 *
 * bca_attend_rope: bca_attend where Q and k_cur are first rotated (token r at
 * position pos0 + r) into staging copies inside the workspace, which the
 * attention then reads; the cached chunks are expected to have been appended
 * with bca_append_chunk_rope. The workspace must hold
 * bca_attend_rope_workspace_bytes() (the bca_attend figure rounded up to 256,
 * plus two [n][H][d] copies in qkv_dtype, each rounded up to 256). Errors as
 * for bca_attend, plus BCA_ERR_INVALID_ARG for rope_base or pos0. */
bca_status bca_append_chunk_rope(bca_cache* cache, int32_t layer, int64_t chunk_id,
                                 int32_t is_ref, const void* k, const void* v, int32_t in_dtype,
                                 double rope_base, int64_t pos0, bca_stream_t stream);

size_t bca_attend_rope_workspace_bytes(const bca_cache* cache, const bca_window_spec* spec);

bca_status bca_attend_rope(const bca_cache* cache, int32_t layer, const bca_window_spec* spec,
                           const void* q, const void* k_cur, const void* v_cur,
                           int32_t qkv_dtype, double rope_base, int64_t pos0, void* o,
                           float* lse, void* workspace, size_t workspace_bytes,
                           bca_stream_t stream);

/* Block-causal attention over a whole sequence of chunks at once (the
 * training form). "WanToFight" review, training Stage 2 (causal adaptation):
 * the model is trained with the same block-causal mask it later streams with,
 * every chunk of a clip attending bidirectionally to itself and to the W
 * chunks before it. Memory prefix: a run of context tokens placed before chunk
 * 0 that every chunk sees (the reference frame of "Matrix-Game 4.0",
 * prerequisite "causal autoregression and KV cache"; a pinned context of sink
 * and memory tokens ahead of the generated chunks in the other pages' memory
 * designs). The prefix has keys and values only, no queries.
 *
 * With C = num_chunks, n = chunk_tokens and P = prefix_tokens, query token
 * r of chunk c (row c*n + r of q) attends to key rows
 *     0 .. P-1                                     (the prefix)
 *     P + c'*n .. P + c'*n + n-1  for max(0, c-W) <= c' <= c,
 * i.e. exactly what bca_attend gives chunk c with the W chunks before it in
 * the ring and the prefix as its reference block (when P = n).
 *
 * Layouts (dense, row-major, qkv_dtype):
 *     q, o : [C*n][H][d]
 *     k, v : [P + C*n][H][d]   prefix rows first, then the chunks in order
 *     lse  : fp32 [C][H][n] (natural log), or NULL
 * qkv_dtype: BCA_F32 or BCA_BF16; head_dim 64 or 128. The work is enqueued on
 * `stream` as attention launches that share the workspace, each followed by a
 * merge launch when its windows are split: with BCA_BF16 one launch per chunk
 * before the window reaches its full length (chunks 0 .. W-1, and chunk W too
 * with a prefix) and one launch for all the remaining chunks, which see the
 * same number of keys; with BCA_F32 one launch per chunk. With BCA_BF16 and
 * num_segments 0, when the clip has at least as many (head, 256-row query
 * tile) units as the device has compute units, the last eight of those
 * launches become one launch, cut where possible on unit boundaries (then
 * nothing is merged and the workspace may be 0 bytes).
 * Errors: BCA_ERR_INVALID_ARG for a NULL or bad spec (non-positive sizes,
 * history < 0, prefix_tokens < 0, num_segments outside [0, 64], non-finite
 * scale), NULL or misaligned buffers (16 bytes; lse 4), or K/V larger than
 * 2 GiB per head's span; BCA_ERR_UNSUPPORTED for another dtype or head_dim;
 * BCA_ERR_WORKSPACE when the workspace is missing, not 256-byte aligned or
 * smaller than bca_attend_sequence_workspace_bytes(); BCA_ERR_HIP for a launch
 * failure (chunks before it may already have been enqueued). */
typedef struct {
  int32_t num_heads;     /* H */
  int32_t head_dim;      /* d */
  int32_t chunk_tokens;  /* n */
  int32_t num_chunks;    /* C */
  int32_t prefix_tokens; /* P >= 0 */
  int32_t history;       /* W >= 0 (W >= C: every earlier chunk) */
  int32_t num_segments;  /* as in bca_window_spec: 0 automatic, G >= 1 segments */
  float scale;           /* softmax scale, usually 1/sqrt(d) */
} bca_sequence_spec;

/* Workspace bytes bca_attend_sequence needs (0 if none, also 0 on a bad spec). */
size_t bca_attend_sequence_workspace_bytes(const bca_sequence_spec* spec, int32_t qkv_dtype);

bca_status bca_attend_sequence(const bca_sequence_spec* spec, const void* q, const void* k,
                               const void* v, int32_t qkv_dtype, void* o, float* lse,
                               void* workspace, size_t workspace_bytes, bca_stream_t stream);

/* Replaying the chunk loop from a captured HIP graph. "Matrix-Game 4.0"
 * summary, prerequisite "FP8 quantisation and CUDA Graph" and experimental
 * results: the per-chunk launches are recorded once and replayed. A graph
 * freezes every launch argument, so what changes from chunk to chunk must
 * live in device memory: here the chunk id, in one int64 the caller owns.
 *
 * bca_append_chunk_dev: bca_append_chunk (not the reference block) whose
 * chunk id is read from *d_chunk_id when the kernels run, writing ring slot
 * (id mod S); a negative id writes nothing. The host cannot see that id, so
 * this call neither checks the order of ids nor updates the host slot table:
 * after the work has run, the caller records it with
 * bca_cache_set_slot_chunk(layer, id mod S, id), as it does after a replay.
 * No rotary form. Errors as for bca_append_chunk, plus BCA_ERR_INVALID_ARG for
 * a NULL or misaligned (8 bytes) d_chunk_id.
 *
 * bca_chunk_counter_advance: *d_chunk_id += 1 in stream order (one thread).
 *
 * bca_attend_replayable: sets *replayable to 1 when a bca_attend of this spec
 * captured now stays right for every later chunk of a stream that appends
 * consecutive ids: the window covers the whole ring (history >= S), every
 * ring slot holds one of the chunks t-S .. t-1 (so an empty slot, and with it
 * any t < S, gives 0), and a requested reference is present. The plan (visible blocks, tiles, work groups) is then the same
 * for every such chunk, and the captured launch reads whatever the slots hold
 * when it runs. Otherwise 0 (a smaller window sees different slots from
 * chunk to chunk). Errors as for bca_attend's checks of cache, layer and spec.
 *
 * bca_attend and bca_append_chunk_dev enqueue kernels only: no allocation,
 * no memset, no synchronisation, so they can be captured. One captured chunk
 * step is: the attends of every layer and denoise step, one
 * bca_append_chunk_dev per layer, one bca_chunk_counter_advance. */
bca_status bca_append_chunk_dev(bca_cache* cache, int32_t layer, const int64_t* d_chunk_id,
                                const void* k, const void* v, int32_t in_dtype,
                                bca_stream_t stream);

bca_status bca_chunk_counter_advance(int64_t* d_chunk_id, bca_stream_t stream);

bca_status bca_attend_replayable(const bca_cache* cache, int32_t layer,
                                 const bca_window_spec* spec, int32_t* replayable);

/* bca_attend for windows smaller than the ring, replayable: the query chunk id
 * is read from *d_q_chunk_id (device int64) when the kernel runs, and the
 * kernel takes the visible ring slots from it: chunks t-W .. t-1 in slots
 * (t-W) mod S .. (t-1) mod S, plus the reference block when use_ref. Valid
 * while the ring holds consecutive ids, as a stream that appends every chunk
 * in order keeps it (bca_append_chunk_dev with the same counter, advanced
 * after the appends). spec->q_chunk_id is the chunk the call is made (or
 * captured) for: the host plans with it and requires every ring slot to hold
 * one of the S chunks before it (no slot empty, hence t >= S). BF16 and 8-bit
 * caches, per-block scales included (each visible block's scales are looked
 * up from the slot it derives); BCA_ERR_UNSUPPORTED for an F32 cache. Other
 * arguments and errors as for bca_attend, plus
 * BCA_ERR_INVALID_ARG for a NULL or misaligned d_q_chunk_id or a ring that
 * does not hold the S chunks before spec->q_chunk_id. */
bca_status bca_attend_dev(const bca_cache* cache, int32_t layer, const bca_window_spec* spec,
                          const int64_t* d_q_chunk_id, const void* q, const void* k_cur,
                          const void* v_cur, int32_t qkv_dtype, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, bca_stream_t stream);

/* Host-side slot table query: chunk id held by ring slot `slot` (0 <= slot < S)
 * of `layer`, -1 if empty. slot == S (with has_ref) reports the reference block
 * (its recorded id, or -1). The table is the ring's bookkeeping of which
 * chunk overwrote which slot (Matrix-Game 4.0 summary, prerequisite "causal
 * autoregression and KV cache": the oldest slot is overwritten in place). */
bca_status bca_cache_slot_chunk(const bca_cache* cache, int32_t layer, int32_t slot,
                                int64_t* chunk_id);

/* Declares the content of a slot without touching device memory, for callers
 * that filled the cache memory themselves (restoring a saved cache). Slot S
 * (with has_ref) is the reference block. chunk_id -1 empties the slot. The
 * layer's newest id is recomputed from the table. For FP8_E4M3_BLOCK and
 * INT8K_FP8V_BLOCK caches the block's scales (the table after the blocks) are
 * part of what the caller restores. */
bca_status bca_cache_set_slot_chunk(bca_cache* cache, int32_t layer, int32_t slot,
                                    int64_t chunk_id);

/* Host-only view of how bca_attend would run (no device work). */
typedef struct {
  int32_t num_visible_blocks; /* including the current chunk                          */
  int32_t visible_blocks[64]; /* physical block per visible block, in key order;
                                 0..S-1 ring slots, S the reference, -1 the current  */
  int64_t visible_chunk_ids[64]; /* chunk id of each visible block (-1: current,
                                    reference: its recorded id)                      */
  int32_t visible_keys;       /* N_k = num_visible_blocks * n                         */
  int32_t q_tiles;            /* query tiles per head                                 */
  int32_t kv_tiles;           /* key tiles per query tile                             */
  int32_t units;              /* H * q_tiles                                          */
  int32_t workgroups;         /* work groups the attention kernel is launched with    */
  int32_t max_pieces;         /* most segments any query tile is split into           */
  int32_t merge;              /* 1 if the log-sum-exp merge kernel runs                */
  size_t workspace_bytes;     /* what this call needs                                 */
} bca_plan_info;

bca_status bca_attend_plan(const bca_cache* cache, int32_t layer, const bca_window_spec* spec,
                           bca_plan_info* out);

/* Static text for a status code. (Library housekeeping; the pages describe no
 * counterpart.) */
const char* bca_status_string(bca_status status);

/* Text of the last error on the calling thread ("" if none). */
const char* bca_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BCA_H */
