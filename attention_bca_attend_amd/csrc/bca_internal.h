// Internal structures shared by the host logic (bca_host.cpp, bca_api.cpp) and the
// HIP kernels (bca_kernels.hip). Not part of the public interface.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/bca.h"

namespace bca {

constexpr int kMaxBlocks = 64;  // ring slots + reference + current chunk
constexpr int kMaxHeadsFp8 = 64;
constexpr int kMaxSegments = 64;
constexpr int kMaxGroups = 8;

// A maximal range of consecutive visible cache keys that sits at one base
// address. Visible cache keys are numbered 0 .. nk_cache-1 in "key order":
// visible ring slots in physical order, then the reference block. A run is a
// range of the head's [(S+R)*n][d] cache matrix.
//
// Key tiles: the first cache_tiles tiles cover the visible cache keys (the
// last one padded with masked keys), the remaining tiles cover the current
// chunk (its own tensor, row stride H*d). No tile mixes the two, so each tile
// is read through one buffer resource.
struct Run {
  int32_t vstart;  // first key of the run in key order
  int32_t len;     // number of keys
  int32_t phys;    // first row in the head's cache matrix
  int32_t moves;   // 1: in a launch over several chunks of a sequence, the run
                   // moves down by chunk_rows rows per chunk (the window);
                   // 0: it stays (a memory prefix)
};

// Consecutive chunks of a bca_attend_sequence launch that share a plan: the
// same keys per unit (T tiles) and the same runs, whose moving runs shift by
// chunk_rows rows per chunk of the group. A launch with groups (ngroups > 0)
// holds chunks whose windows differ in length (the chunks before the window
// is full); its units are numbered chunk by chunk, group after group.
struct UnitGroup {
  int64_t iter0;        // first tile iteration of the group
  int32_t units0;       // first unit of the group
  int32_t T;            // key tiles per unit
  int32_t cache_tiles;  // key tiles over the cache keys
  int32_t nk_cache;     // visible cache keys
  int32_t run0, nruns;  // the group's runs: runs[run0 .. run0 + nruns)
  int32_t chunk0;       // the group's first chunk, counted from the launch's first
  int32_t pad;
};

// Kernel families; each has fixed tile sizes.
enum class Kern : int { F32 = 0, BF16 = 1, FP8 = 2 };

struct TileShape {
  int bm;  // query rows per work group
  int bn;  // keys per tile
};

inline TileShape tile_shape(Kern k) {
  switch (k) {
    case Kern::F32: return {64, 32};
    case Kern::BF16: return {256, 64};
    case Kern::FP8: return {256, 64};
  }
  return {128, 64};
}

// What one bca_attend call does, as resolved on the host.
struct Plan {
  Kern kern;
  int32_t seq;                      // 1: a bca_attend_sequence launch (token-major cache rows)
  int32_t devt;                     // 1: visible slots derived on the device (bca_attend_dev)
  int32_t blk;                      // 1: per-block 8-bit cache (tiles aligned to blocks)
  int32_t i8k;                      // 1: INT8K_FP8V_BLOCK (K int8, Q K^T on int8 MFMA)
  int32_t tpb;                      // key tiles per block when blk
  int32_t nvis;                     // visible blocks, current included
  int32_t vis_block[kMaxBlocks];    // physical block (S = reference, -1 = current)
  int64_t vis_id[kMaxBlocks];
  int32_t nruns;
  Run runs[kMaxBlocks];
  int32_t nk;                       // visible keys (cache + current)
  int32_t nk_cache;                 // visible cache keys
  int32_t cache_tiles;              // key tiles over the cache keys
  int32_t bm, bn;
  int32_t q_tiles, kv_tiles, units; // units = H * q_tiles
  int32_t wgs;                      // work groups (P)
  int32_t jmax;                     // most work groups any unit is split over
  int32_t spw;                      // partial-output slots per work group (1 or 2)
  int32_t merge;                    // 1: some unit is split over work groups
  int32_t ngroups;                  // > 0: units of different lengths (see UnitGroup)
  int64_t iters;                    // tile iterations of the launch
  UnitGroup grp[kMaxGroups];
  size_t stage_off;                 // fp8 cache: offset of the current-chunk staging copy
  size_t ws_bytes;                  // workspace this call needs
};

// Arguments of the attention kernels (passed by value as kernel arguments).
struct AttnArgs {
  const void* q;      // [n][H][d]
  const void* kcur;   // [n][H][d]; fp8 cache: the staging copy [H][n][d] e4m3
  const void* vcur;   // [n][H][d]; fp8 cache: the staging copy [H][n][d] e4m3
  const void* kcur_in;  // fp8 cache: the caller's bf16 K of the chunk [n][H][d]
  const void* vcur_in;
  const void* kc;     // this layer's K blocks: [H][S+R][n][d]
  const void* vc;     // this layer's V blocks
  void* o;            // [n][H][d]
  float* lse;         // [H][n] or null
  float* part_o;      // [P][spw][bm][d]: fp32 (fp32 path), or fp16 scaled per row
                      // and stored as the lanes hold them (bf16, 8-bit paths)
  float* part_lse;    // [P][spw][bm]
  int32_t* part_exp;  // [P][spw][bm]: the fp16 partials' row exponents (merge_lanes_kernel)
  int64_t cache_head_elems;  // elements between heads' first cache rows: (S+R)*n*d for the
                             // ring, d for a token-major sequence [rows][H][d]
  int64_t cache_span_elems;  // elements one head's cache rows span (buffer resource size)
  int32_t cache_row_elems;   // elements between consecutive cache rows: d (ring), H*d (sequence)
  int32_t n, H, nk_cache, cache_tiles, T, QT, units, P, spw;
  float scale;        // softmax scale
  float scale_log2;   // scale * log2(e)
  int32_t xcd_remap;  // 1: spread work-group ids so each XCD gets a contiguous range
  // One launch may cover several consecutive chunks of a sequence that share
  // a plan: unit u is unit u % upc of chunk u / upc, whose q, k_cur, v_cur and
  // o start chunk_elems elements further per chunk, lse chunk_lse floats, and
  // whose moving runs start chunk_rows rows further. upc = units otherwise.
  int32_t upc;
  // Query chunk id read on the device (bca_attend_dev): the kernel derives
  // the visible ring slots from *dev_t, W = dev_W and S = dev_S (the ring
  // holding consecutive ids), plus the reference block when dev_ref.
  const int64_t* dev_t;
  int32_t dev_W, dev_S, dev_ref;
  int32_t chunk_rows;
  int64_t chunk_elems;
  int64_t chunk_lse;
  int32_t nruns;
  Run runs[kMaxBlocks];
  float k_scale[kMaxHeadsFp8];  // fp8 cache: dequantisation scale per head
  float v_scale[kMaxHeadsFp8];
  // Per-block caches: every visible cache block is its own run, padded to tpb
  // whole key tiles; ksc/vsc are the layer's scale tables [S+R][H], cur_sc the
  // current chunk's scales [K|V][H]; vis_blk the physical block of each of the
  // nvis_cache visible cache blocks.
  int32_t blk, i8k, tpb, nvis_cache;
  // Grouped sequence launches: ngroups > 0 groups of units (UnitGroup), iters
  // tile iterations in all; otherwise every unit has T tiles and the runs,
  // nk_cache and cache_tiles above.
  int32_t ngroups;
  int64_t iters;
  UnitGroup grp[kMaxGroups];
  const float* ksc;
  const float* vsc;
  const float* cur_sc;
  int8_t vis_blk[kMaxBlocks];
};

struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  const int32_t* part_exp;  // fp16 partials only
  void* o;
  float* lse;
  int32_t n, H, T, QT, units, P, spw, bm;
  int32_t upc;          // units per chunk (see AttnArgs)
  int64_t chunk_elems;  // o elements per chunk
  int64_t chunk_lse;    // lse floats per chunk
  int32_t ngroups;      // grouped launch (see AttnArgs)
  int64_t iters;
  UnitGroup grp[kMaxGroups];
};

struct AppendArgs {
  const void* k;   // [n][H][d]
  const void* v;
  void* kdst;      // this layer's K blocks, block `blk`
  void* vdst;
  int64_t head_stride_elems;  // (S+R)*n*d
  int32_t n, H;
  float k_scale[kMaxHeadsFp8];  // fp8 cache only
  float v_scale[kMaxHeadsFp8];
  // Device-side chunk id (graph replay): when set, kdst/vdst are the layer's
  // block 0 and the kernels read the id when they run and write block
  // (id mod slots), block_elems elements per block; a negative id writes
  // nothing.
  const int64_t* dev_chunk;
  int32_t slots;
  int64_t block_elems;
  // Scales from device memory (per-block caches, and the current chunk's copy):
  // ksc/vsc point at [blocks][H] tables; the block is host_blk, or
  // (id mod slots) with dev_chunk. append_amax_kernel writes them first.
  int32_t dev_scales;
  int32_t k_int8;          // 1: K codes are int8 (scale = max |x| / 127), V stays e4m3
  int32_t host_blk;
  float* ksc;
  float* vsc;
  int32_t rope;            // 1: rotate K (rotary embedding) before it is stored
  double rope_log2_base;   // log2 of the rotary base
  int64_t rope_pos0;       // position of the chunk's token 0
};

// Rotary embedding of a chunk's Q and K into staging copies (same layout).
struct RopeStageArgs {
  const void* src[2];  // q, k_cur: [n][H][d]
  void* dst[2];
  int32_t n, H;
  double log2_base;
  int64_t pos0;
};

// Launchers (bca_kernels.hip). They return the HIP error code (0 = success).
int launch_attention(const Plan& plan, const AttnArgs& args, int head_dim, void* stream);
int launch_append(bca_dtype in, bca_dtype kv, int head_dim, const AppendArgs& args,
                  void* stream);
int launch_rope_stage(bca_dtype dt, int head_dim, const RopeStageArgs& args, void* stream);
int launch_counter_advance(int64_t* counter, void* stream);
// Compute units of the current device, or 0 when it cannot be queried.
int device_compute_units();
// Device address of the current device's bca_attend_noalloc scratch
// (BCA_NOALLOC_SCRATCH_BYTES bytes), looked up on the first call per device.
// Returns the HIP error code (0 = success).
int noalloc_scratch(void** out);

}  // namespace bca
