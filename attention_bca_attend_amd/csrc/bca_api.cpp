// bca_api.cpp — the C interface of include/bca.h: cache handle, slot table,
// window resolution, work planning, argument validation and kernel launches.
//
// Pure host C++: the only device work is the kernels bca_kernels.hip launches.
//
// Sources for the semantics (the web pages this library is built from):
//  - "WanToFight: Real-Time Generative Game Engine for Multi-Player Combat
//    Interaction" (xllm-io review), section 3 model components table
//    (Block-Causal Attention: bidirectional in the chunk, across chunks the
//    current one and the previous 2; Rolling KV Cache: the last 2 chunks,
//    updated after each chunk) and section 5, code analysis (KV cached after the
//    chunk is generated).
//  - "Matrix-Game 4.0: Harnessing Video Models for Real-Time Playable Game
//    Worlds" (paper summary), prerequisite "causal autoregression and KV cache"
//    (recent window of 20 chunks plus a reference frame; the ring buffer writes
//    the newest chunk over the oldest slot in place; split-window attention
//    with a log-sum-exp merge) and "technical novelty" (7 intervals, 8-bit KV).
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "bca_internal.h"

using namespace bca;

struct bca_cache {
  bca_cache_desc d;
  char* mem = nullptr;
  size_t bytes = 0;
  std::vector<int64_t> slot;       // [L][S] chunk id per ring slot, -1 empty
  std::vector<int64_t> newest;     // [L] newest ring chunk id, -1 none
  std::vector<int64_t> ref_id;     // [L] recorded id of the reference chunk
  std::vector<uint8_t> ref_valid;  // [L]
  std::vector<float> k_scale;      // [L][H] fp8 dequantisation scales
  std::vector<float> v_scale;
  int num_cus = 0;
};

namespace {

thread_local std::string g_err;

bca_status fail(bca_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
bca_status fail(bca_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

size_t elem_size(int32_t dt) {
  switch (dt) {
    case BCA_F32: return 4;
    case BCA_BF16: return 2;
    case BCA_FP8_E4M3: return 1;
    case BCA_FP8_E4M3_BLOCK: return 1;
    case BCA_INT8K_FP8V_BLOCK: return 1;
  }
  return 0;
}

// Caches with one scale per (layer, block, head), taken from each appended chunk.
bool is_blk(int32_t kv) { return kv == BCA_FP8_E4M3_BLOCK || kv == BCA_INT8K_FP8V_BLOCK; }
// 8-bit caches (served by the fp8 attention kernel).
bool is_fp8(int32_t kv) { return kv == BCA_FP8_E4M3 || is_blk(kv); }

bool desc_ok(const bca_cache_desc* d, std::string* why) {
  auto bad = [&](const char* m) {
    if (why) *why = m;
    return false;
  };
  if (!d) return bad("desc is NULL");
  if (d->num_layers < 1) return bad("num_layers must be >= 1");
  if (d->num_heads < 1) return bad("num_heads must be >= 1");
  if (d->head_dim != 64 && d->head_dim != 128) return bad("head_dim must be 64 or 128");
  if (d->chunk_tokens < 1) return bad("chunk_tokens must be >= 1");
  if (d->ring_slots < 1 || d->ring_slots > kMaxBlocks - 2)
    return bad("ring_slots must be in [1, 62]");
  if (d->has_ref != 0 && d->has_ref != 1) return bad("has_ref must be 0 or 1");
  if (elem_size(d->kv_dtype) == 0) return bad("kv_dtype is not a bca_dtype");
  if (is_fp8(d->kv_dtype)) {
    if (d->num_heads > kMaxHeadsFp8) return bad("8-bit caches support at most 64 heads");
    if (d->head_dim != 128) return bad("8-bit caches need head_dim 128");
  }
  // keys per head (all blocks plus the current chunk) must fit int32 with room
  const int64_t blocks = (int64_t)d->ring_slots + d->has_ref + 1;
  if (blocks * (int64_t)d->chunk_tokens > (int64_t)1 << 30) return bad("chunk_tokens too large");
  // the kernels address one head's cache blocks, and one chunk's q/k/v/o
  // rows, with 32-bit byte offsets
  const int64_t limit = (int64_t)INT32_MAX - 4096;
  const int64_t head_bytes = ((int64_t)d->ring_slots + d->has_ref) * d->chunk_tokens *
                             d->head_dim * (int64_t)elem_size(d->kv_dtype);
  const int64_t qkv_es = d->kv_dtype == BCA_F32 ? 4 : 2;
  const int64_t chunk_bytes = (int64_t)d->chunk_tokens * d->num_heads * d->head_dim * qkv_es;
  if (head_bytes > limit) return bad("one head's cache blocks exceed 2 GiB");
  if (chunk_bytes > limit) return bad("one chunk's q/k/v rows exceed 2 GiB");
  return true;
}

// Bytes of one layer's K (or V) blocks: H * (S+R) * n * d elements.
size_t half_layer_bytes(const bca_cache_desc& d) {
  return (size_t)d.num_heads * (size_t)(d.ring_slots + d.has_ref) * (size_t)d.chunk_tokens *
         (size_t)d.head_dim * elem_size(d.kv_dtype);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Per-block caches: the scale table after the blocks, fp32 [L][K|V][S+R][H].
size_t block_scale_bytes(const bca_cache_desc& d) {
  if (!is_blk(d.kv_dtype)) return 0;
  const size_t n = (size_t)d.num_layers * 2 * (d.ring_slots + d.has_ref) * d.num_heads * 4;
  return (n + 255) & ~(size_t)255;
}

// Key tiles of one block: per-block caches pad every visible block to whole
// tiles, so that each tile has one block's scales.
int block_tiles(const bca_cache_desc& d) { return (d.chunk_tokens + 63) / 64; }

bool layer_ok(const bca_cache* c, int32_t layer) {
  return layer >= 0 && layer < c->d.num_layers;
}

Kern kernel_for(int32_t qkv, int32_t kv) {
  if (qkv == BCA_F32 && kv == BCA_F32) return Kern::F32;
  if (qkv == BCA_BF16 && kv == BCA_BF16) return Kern::BF16;
  return Kern::FP8;
}

bool pair_supported(int32_t qkv, int32_t kv) {
  return (qkv == BCA_F32 && kv == BCA_F32) || (qkv == BCA_BF16 && kv == BCA_BF16) ||
         (qkv == BCA_BF16 && is_fp8(kv));
}

int wgs_per_cu(Kern k) {
  // resident work groups per CU (LDS and register limited)
  switch (k) {
    case Kern::F32: return 4;
    case Kern::BF16: return 1;
    case Kern::FP8: return 1;
  }
  return 1;
}

int compute_units(const bca_cache* c) { return c->num_cus > 0 ? c->num_cus : 256; }

// First work group whose iteration range contains iteration x when I
// iterations are cut into P consecutive ranges [floor(w I / P), floor((w+1) I / P)).
int64_t first_wg(int64_t x, int64_t I, int64_t P) { return ((x + 1) * P + I - 1) / I - 1; }

// Partial-output slots a unit of T tiles needs when I = units*T iterations
// are cut into P ranges (the largest number of ranges any unit touches).
int32_t pieces_bound(int64_t units, int64_t T, int64_t P) {
  int64_t I = units * T, worst = 1;
  for (int64_t u = 0; u < units; ++u) {
    int64_t a = first_wg(u * T, I, P), b = first_wg((u + 1) * T - 1, I, P);
    if (b - a + 1 > worst) worst = b - a + 1;
  }
  return (int32_t)worst;
}

// Work groups of a launch. num_segments = G >= 1: every unit in G equal
// segments. Automatic: when the units fit on the device, every unit in the
// same number of equal segments, as many as fit (no work group then crosses
// a unit boundary, and each unit has the fewest partial outputs to merge);
// otherwise one range of tile iterations per resident work group
// ("stream-K").
// Work groups for a stream-K cut of I iterations over units whose first
// iterations unit_first(u) (u = 0 .. units, unit_first(units) = I) are given:
// among the counts from target down to 97 % of it, the one that leaves the
// fewest units split across work groups (each split unit costs partial
// outputs and their merge; 3 % fewer work groups cost at most 3 % more
// tiles per group). A cut whose ranges all end on unit boundaries needs no
// merge at all.
template <typename First>
int64_t fewest_split_wgs(int64_t I, int64_t units, int64_t target, First unit_first) {
  const int64_t hi = std::max<int64_t>(1, std::min(I, target));
  const int64_t lo = std::max<int64_t>(1, hi - hi * 3 / 100);
  int64_t best = hi, best_split = -1;
  for (int64_t P = hi; P >= lo; --P) {
    int64_t split = 0;
    for (int64_t u = 0; u < units; ++u)
      split += first_wg(unit_first(u + 1) - 1, I, P) != first_wg(unit_first(u), I, P);
    if (best_split < 0 || split < best_split) {
      best = P;
      best_split = split;
    }
    if (split == 0) break;
  }
  return best;
}

int64_t choose_wgs_on(int cus, Kern k, int64_t units, int64_t T, int32_t G) {
  const int64_t I = units * T;
  if (G >= 1) return units * std::min<int64_t>(G, T);
  const int64_t target = (int64_t)cus * wgs_per_cu(k);
  if (units <= target) return units * std::min<int64_t>(T, target / units);
  return fewest_split_wgs(I, units, target, [T](int64_t u) { return u * T; });
}

int64_t choose_wgs(const bca_cache* c, Kern k, int64_t units, int64_t T, int32_t G) {
  return choose_wgs_on(compute_units(c), k, units, T, G);
}

// fp8 cache: the current chunk's K and V quantised to e4m3, [H][n][d] each,
// 256-byte aligned regions.
size_t fp8_stage_bytes(const bca_cache_desc& d) {
  const size_t one = ((size_t)d.num_heads * d.chunk_tokens * d.head_dim + 255) & ~(size_t)255;
  return 2 * one;
}

// Per-block caches: the current chunk's own scales [K|V][H] after its copy.
size_t cur_scale_bytes(const bca_cache_desc& d) {
  return ((size_t)2 * d.num_heads * 4 + 255) & ~(size_t)255;
}

// Per-block scale table of one layer's K (kv 0) or V (kv 1): [S+R][H].
float* block_scales(const bca_cache* c, int32_t layer, int kv) {
  const bca_cache_desc& d = c->d;
  float* t = reinterpret_cast<float*>(c->mem + 2 * (size_t)d.num_layers * half_layer_bytes(d));
  return t + ((size_t)layer * 2 + kv) * (d.ring_slots + d.has_ref) * d.num_heads;
}

// Partial-output slots per work group: 1 when every work group's range lies
// within one unit (each unit cut into P / units equal ranges), else 2 (a range
// can end one unit and start the next).
int32_t slots_per_wg(int64_t units, int64_t P) { return (P >= units && P % units == 0) ? 1 : 2; }

// Bytes of part_o [P][spw][bm][d] (sized for fp32), then part_lse [P][spw][bm]
// fp32, each region 256-byte aligned. The fp16 partials of the bf16 and 8-bit
// paths fill the first half of part_o; their row exponents [P][spw][bm]
// (int32) follow them in the second half (part_exp_offset). The fp32 path
// fills part_o with fp32.
size_t part_o_bytes(int64_t P, int32_t spw, int bm, int d) {
  return ((size_t)P * spw * bm * d * 4 + 255) & ~(size_t)255;
}
size_t part_exp_offset(int64_t P, int32_t spw, int bm, int d) {
  return (size_t)P * spw * bm * d * 2;
}
size_t partial_bytes(int64_t P, int32_t spw, int bm, int d) {
  const size_t pl = (size_t)P * spw * bm * 4;
  return part_o_bytes(P, spw, bm, d) + ((pl + 255) & ~(size_t)255);
}

// Window resolution and planning shared by bca_attend, bca_attend_plan and
// bca_attend_workspace_bytes. Validates everything except device pointers.
bca_status make_plan(const bca_cache* c, int32_t layer, const bca_window_spec* s,
                     int32_t qkv_dtype, Plan& p) {
  std::memset(&p, 0, sizeof p);
  if (!c) return fail(BCA_ERR_INVALID_ARG, "cache is NULL");
  if (!s) return fail(BCA_ERR_INVALID_ARG, "spec is NULL");
  if (!layer_ok(c, layer))
    return fail(BCA_ERR_INVALID_ARG, "layer %d out of range [0, %d)", layer, c->d.num_layers);
  const bca_cache_desc& d = c->d;
  const int S = d.ring_slots, n = d.chunk_tokens;
  if (s->q_chunk_id < 0) return fail(BCA_ERR_INVALID_ARG, "q_chunk_id must be >= 0");
  if (s->history < 0 || s->history > S)
    return fail(BCA_ERR_INVALID_ARG, "history %d must be in [0, ring_slots=%d]", s->history, S);
  if (s->use_ref != 0 && s->use_ref != 1)
    return fail(BCA_ERR_INVALID_ARG, "use_ref must be 0 or 1");
  if (s->use_ref && !d.has_ref)
    return fail(BCA_ERR_INVALID_ARG, "use_ref set but the cache has no reference block");
  if (s->num_segments < 0 || s->num_segments > kMaxSegments)
    return fail(BCA_ERR_INVALID_ARG, "num_segments must be in [0, 64]");
  if (!std::isfinite(s->scale)) return fail(BCA_ERR_INVALID_ARG, "scale must be finite");
  if (elem_size(qkv_dtype) == 0)
    return fail(BCA_ERR_INVALID_ARG, "qkv_dtype is not a bca_dtype");
  if (!pair_supported(qkv_dtype, d.kv_dtype))
    return fail(BCA_ERR_UNSUPPORTED, "no kernel for qkv dtype %d with cache dtype %d",
                qkv_dtype, d.kv_dtype);
  const int64_t t = s->q_chunk_id, W = s->history;
  const int64_t newest = c->newest[layer];
  // Residency: chunk c is overwritten only by a chunk c' = c + k*S (k >= 1) that
  // was appended later. If the newest ring id is below t - W + S, every such
  // c' is >= c + S > newest for window chunks c >= t - W, so the window is intact.
  if (newest >= 0 && newest >= t - W + S)
    return fail(BCA_ERR_OUT_OF_ORDER,
                "window of chunk %lld (history %lld) may be overwritten: newest ring chunk "
                "is %lld with %d slots",
                (long long)t, (long long)W, (long long)newest, S);

  // a1: visible blocks, resolved from the slot table's chunk ids
  p.nvis = 0;
  for (int sl = 0; sl < S; ++sl) {
    int64_t cid = c->slot[(size_t)layer * S + sl];
    if (cid >= 0 && cid >= t - W && cid <= t - 1) {
      p.vis_block[p.nvis] = sl;
      p.vis_id[p.nvis++] = cid;
    }
  }
  if (s->use_ref && c->ref_valid[layer]) {
    p.vis_block[p.nvis] = S;
    p.vis_id[p.nvis++] = c->ref_id[layer];
  }
  p.vis_block[p.nvis] = -1;
  p.vis_id[p.nvis++] = -1;
  p.nk = p.nvis * n;

  // runs of the cache part: consecutive physical blocks share one run
  // (per-block caches: one run per block, each padded to whole key tiles)
  p.nruns = 0;
  p.blk = is_blk(d.kv_dtype) ? 1 : 0;
  p.i8k = d.kv_dtype == BCA_INT8K_FP8V_BLOCK ? 1 : 0;
  p.tpb = block_tiles(d);
  if (p.blk) {
    for (int i = 0; i + 1 < p.nvis; ++i) {
      Run r;
      r.vstart = i * p.tpb * 64;
      r.len = n;
      r.phys = p.vis_block[i] * n;
      r.moves = 0;
      p.runs[p.nruns++] = r;
    }
  }
  for (int i = 0; !p.blk && i + 1 < p.nvis; ++i) {
    const int b = p.vis_block[i];
    if (p.nruns > 0 && p.runs[p.nruns - 1].phys + p.runs[p.nruns - 1].len == b * n) {
      p.runs[p.nruns - 1].len += n;
      continue;
    }
    Run r;
    r.vstart = i * n;
    r.len = n;
    r.phys = b * n;
    r.moves = 0;
    p.runs[p.nruns++] = r;
  }
  p.nk_cache = p.blk ? (p.nvis - 1) * p.tpb * 64 : (p.nvis - 1) * n;

  // a3: work planning. Every query row of the chunk sees the same keys, so all
  // units (head, query tile) have the same number of key tiles T. The
  // units*T tile iterations are cut into P equal consecutive ranges, one per
  // work group; a unit that spans several ranges is computed as several
  // segments whose partial results are merged by log-sum-exp. With
  // num_segments = G >= 1, P = units*min(G, T) makes every unit exactly G
  // segments of near-equal length.
  p.kern = kernel_for(qkv_dtype, d.kv_dtype);
  TileShape ts = tile_shape(p.kern);
  p.bm = ts.bm;
  p.bn = ts.bn;
  p.q_tiles = (n + p.bm - 1) / p.bm;
  p.cache_tiles = (p.nk_cache + p.bn - 1) / p.bn;
  p.kv_tiles = p.cache_tiles + (n + p.bn - 1) / p.bn;
  p.units = d.num_heads * p.q_tiles;
  p.wgs = (int32_t)choose_wgs(c, p.kern, p.units, p.kv_tiles, s->num_segments);
  p.jmax = pieces_bound(p.units, p.kv_tiles, p.wgs);
  p.merge = p.jmax > 1 ? 1 : 0;
  p.spw = slots_per_wg(p.units, p.wgs);
  p.ws_bytes = p.merge ? partial_bytes(p.wgs, p.spw, p.bm, d.head_dim) : 0;
  p.stage_off = p.ws_bytes;
  if (p.kern == Kern::FP8) p.ws_bytes += fp8_stage_bytes(d);
  if (p.blk) p.ws_bytes += cur_scale_bytes(d);
  return BCA_OK;
}

}  // namespace

extern "C" {

size_t bca_cache_bytes(const bca_cache_desc* desc) {
  std::string why;
  if (!desc_ok(desc, &why)) return 0;
  return 2 * (size_t)desc->num_layers * half_layer_bytes(*desc) + block_scale_bytes(*desc);
}

bca_status bca_cache_create(const bca_cache_desc* desc, void* dev_mem, size_t bytes,
                            bca_cache** out) {
  std::string why;
  if (!out) return fail(BCA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!desc_ok(desc, &why)) return fail(BCA_ERR_INVALID_ARG, "%s", why.c_str());
  size_t need = bca_cache_bytes(desc);
  if (!dev_mem) return fail(BCA_ERR_INVALID_ARG, "dev_mem is NULL");
  if (!aligned(dev_mem, 256)) return fail(BCA_ERR_INVALID_ARG, "dev_mem not 256-byte aligned");
  if (bytes < need)
    return fail(BCA_ERR_INVALID_ARG, "cache memory %zu bytes < required %zu", bytes, need);
  bca_cache* c = new (std::nothrow) bca_cache;
  if (!c) return fail(BCA_ERR_INVALID_ARG, "out of host memory");
  c->d = *desc;
  c->mem = static_cast<char*>(dev_mem);
  c->bytes = bytes;
  const size_t L = desc->num_layers, S = desc->ring_slots, H = desc->num_heads;
  c->slot.assign(L * S, -1);
  c->newest.assign(L, -1);
  c->ref_id.assign(L, -1);
  c->ref_valid.assign(L, 0);
  c->k_scale.assign(L * H, 1.0f);
  c->v_scale.assign(L * H, 1.0f);
  c->num_cus = device_compute_units();
  *out = c;
  g_err.clear();
  return BCA_OK;
}

bca_status bca_cache_destroy(bca_cache* cache) {
  delete cache;
  return BCA_OK;
}

bca_status bca_cache_set_kv_scales(bca_cache* c, int32_t layer, const float* k_scale,
                                   const float* v_scale) {
  if (!c) return fail(BCA_ERR_INVALID_ARG, "cache is NULL");
  if (is_blk(c->d.kv_dtype))
    return fail(BCA_ERR_UNSUPPORTED, "per-block caches take their scales from the appends");
  if (c->d.kv_dtype != BCA_FP8_E4M3)
    return fail(BCA_ERR_INVALID_ARG, "scales apply to FP8_E4M3 caches only");
  if (!layer_ok(c, layer)) return fail(BCA_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (!k_scale || !v_scale) return fail(BCA_ERR_INVALID_ARG, "scale array is NULL");
  const int H = c->d.num_heads;
  for (int h = 0; h < H; ++h) {
    if (!(std::isfinite(k_scale[h]) && k_scale[h] > 0.f && std::isfinite(v_scale[h]) &&
          v_scale[h] > 0.f))
      return fail(BCA_ERR_INVALID_ARG, "scale of head %d is not positive and finite", h);
  }
  for (int h = 0; h < H; ++h) {
    c->k_scale[(size_t)layer * H + h] = k_scale[h];
    c->v_scale[(size_t)layer * H + h] = v_scale[h];
  }
  // chunks stored under the old scales no longer decode correctly
  const int S = c->d.ring_slots;
  for (int s = 0; s < S; ++s) c->slot[(size_t)layer * S + s] = -1;
  c->newest[layer] = -1;
  c->ref_valid[layer] = 0;
  c->ref_id[layer] = -1;
  g_err.clear();
  return BCA_OK;
}

}  // extern "C"

namespace {

// Rotary embedding parameters of one call (bca_append_chunk_rope / bca_attend_rope).
struct RopeArg {
  double log2_base;
  int64_t pos0;
};

bca_status check_rope(double base, int64_t pos0) {
  if (!std::isfinite(base) || !(base > 0.0))
    return fail(BCA_ERR_INVALID_ARG, "rope_base must be finite and > 0");
  if (pos0 < 0) return fail(BCA_ERR_INVALID_ARG, "rope position must be >= 0");
  return BCA_OK;
}

bca_status append_impl(bca_cache* c, int32_t layer, int64_t chunk_id, int32_t is_ref,
                       const void* k, const void* v, int32_t in_dtype, bca_stream_t stream,
                       const RopeArg* rope) {
  if (!c) return fail(BCA_ERR_INVALID_ARG, "cache is NULL");
  if (!layer_ok(c, layer))
    return fail(BCA_ERR_INVALID_ARG, "layer %d out of range [0, %d)", layer, c->d.num_layers);
  if (chunk_id < 0) return fail(BCA_ERR_INVALID_ARG, "chunk_id must be >= 0");
  if (is_ref != 0 && is_ref != 1) return fail(BCA_ERR_INVALID_ARG, "is_ref must be 0 or 1");
  if (is_ref && !c->d.has_ref)
    return fail(BCA_ERR_INVALID_ARG, "is_ref set but the cache has no reference block");
  if (!k || !v) return fail(BCA_ERR_INVALID_ARG, "k or v is NULL");
  if (!aligned(k, 16) || !aligned(v, 16))
    return fail(BCA_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  if (elem_size(in_dtype) == 0) return fail(BCA_ERR_INVALID_ARG, "in_dtype is not a bca_dtype");
  const int32_t kv = c->d.kv_dtype;
  bool ok = (in_dtype == BCA_F32 && kv == BCA_F32) || (in_dtype == BCA_BF16 && kv == BCA_BF16) ||
            (in_dtype == BCA_BF16 && is_fp8(kv));
  if (!ok)
    return fail(BCA_ERR_UNSUPPORTED, "cannot append dtype %d into a cache of dtype %d",
                in_dtype, kv);
  const int S = c->d.ring_slots;
  if (!is_ref && chunk_id < c->newest[layer])
    return fail(BCA_ERR_OUT_OF_ORDER, "chunk %lld appended after chunk %lld on layer %d",
                (long long)chunk_id, (long long)c->newest[layer], layer);
  // the oldest chunk's slot is overwritten in place: slot = id mod S
  const int blk = is_ref ? S : (int)(chunk_id % S);
  const size_t es = elem_size(kv);
  const bca_cache_desc& d = c->d;
  const size_t block_elems = (size_t)d.chunk_tokens * d.head_dim;
  char* layer_k = c->mem + 2 * (size_t)layer * half_layer_bytes(d);
  char* layer_v = layer_k + half_layer_bytes(d);
  AppendArgs a;
  std::memset(&a, 0, sizeof a);
  a.k = k;
  a.v = v;
  a.kdst = layer_k + (size_t)blk * block_elems * es;
  a.vdst = layer_v + (size_t)blk * block_elems * es;
  a.head_stride_elems = (int64_t)(S + d.has_ref) * (int64_t)block_elems;
  a.n = d.chunk_tokens;
  a.H = d.num_heads;
  if (kv == BCA_FP8_E4M3)
    for (int h = 0; h < d.num_heads; ++h) {
      a.k_scale[h] = c->k_scale[(size_t)layer * d.num_heads + h];
      a.v_scale[h] = c->v_scale[(size_t)layer * d.num_heads + h];
    }
  if (is_blk(kv)) {
    // with rotation, the block's K scale is taken over the rotated rows
    a.dev_scales = 1;
    a.k_int8 = kv == BCA_INT8K_FP8V_BLOCK ? 1 : 0;
    a.host_blk = blk;
    a.ksc = block_scales(c, layer, 0);
    a.vsc = block_scales(c, layer, 1);
  }
  if (rope) {
    a.rope = 1;
    a.rope_log2_base = rope->log2_base;
    a.rope_pos0 = rope->pos0;
  }
  int err = launch_append((bca_dtype)in_dtype, (bca_dtype)kv, d.head_dim, a, (void*)stream);
  if (err != 0) return fail(BCA_ERR_HIP, "append kernel launch failed (hip error %d)", err);
  if (is_ref) {
    c->ref_valid[layer] = 1;
    c->ref_id[layer] = chunk_id;
  } else {
    c->slot[(size_t)layer * S + blk] = chunk_id;
    c->newest[layer] = chunk_id;
  }
  g_err.clear();
  return BCA_OK;
}

}  // namespace

extern "C" {

bca_status bca_append_chunk_dev(bca_cache* c, int32_t layer, const int64_t* d_chunk_id,
                                const void* k, const void* v, int32_t in_dtype,
                                bca_stream_t stream) {
  if (!c) return fail(BCA_ERR_INVALID_ARG, "cache is NULL");
  if (!layer_ok(c, layer))
    return fail(BCA_ERR_INVALID_ARG, "layer %d out of range [0, %d)", layer, c->d.num_layers);
  if (!d_chunk_id || !aligned(d_chunk_id, 8))
    return fail(BCA_ERR_INVALID_ARG, "d_chunk_id must be a non-NULL, 8-byte aligned pointer");
  if (!k || !v) return fail(BCA_ERR_INVALID_ARG, "k or v is NULL");
  if (!aligned(k, 16) || !aligned(v, 16))
    return fail(BCA_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  if (elem_size(in_dtype) == 0) return fail(BCA_ERR_INVALID_ARG, "in_dtype is not a bca_dtype");
  const int32_t kv = c->d.kv_dtype;
  bool ok = (in_dtype == BCA_F32 && kv == BCA_F32) || (in_dtype == BCA_BF16 && kv == BCA_BF16) ||
            (in_dtype == BCA_BF16 && is_fp8(kv));
  if (!ok)
    return fail(BCA_ERR_UNSUPPORTED, "cannot append dtype %d into a cache of dtype %d",
                in_dtype, kv);
  const bca_cache_desc& d = c->d;
  const size_t block_elems = (size_t)d.chunk_tokens * d.head_dim;
  char* layer_k = c->mem + 2 * (size_t)layer * half_layer_bytes(d);
  AppendArgs a;
  std::memset(&a, 0, sizeof a);
  a.k = k;
  a.v = v;
  a.kdst = layer_k;  // block 0; the kernels add (id mod S) blocks
  a.vdst = layer_k + half_layer_bytes(d);
  a.head_stride_elems = (int64_t)(d.ring_slots + d.has_ref) * (int64_t)block_elems;
  a.n = d.chunk_tokens;
  a.H = d.num_heads;
  a.dev_chunk = d_chunk_id;
  a.slots = d.ring_slots;
  a.block_elems = (int64_t)block_elems;
  if (kv == BCA_FP8_E4M3)
    for (int h = 0; h < d.num_heads; ++h) {
      a.k_scale[h] = c->k_scale[(size_t)layer * d.num_heads + h];
      a.v_scale[h] = c->v_scale[(size_t)layer * d.num_heads + h];
    }
  if (is_blk(kv)) {
    a.dev_scales = 1;
    a.k_int8 = kv == BCA_INT8K_FP8V_BLOCK ? 1 : 0;
    a.ksc = block_scales(c, layer, 0);
    a.vsc = block_scales(c, layer, 1);
  }
  int err = launch_append((bca_dtype)in_dtype, (bca_dtype)kv, d.head_dim, a, (void*)stream);
  if (err != 0) return fail(BCA_ERR_HIP, "append kernel launch failed (hip error %d)", err);
  g_err.clear();
  return BCA_OK;
}

bca_status bca_chunk_counter_advance(int64_t* d_chunk_id, bca_stream_t stream) {
  if (!d_chunk_id || !aligned(d_chunk_id, 8))
    return fail(BCA_ERR_INVALID_ARG, "d_chunk_id must be a non-NULL, 8-byte aligned pointer");
  int err = launch_counter_advance(d_chunk_id, (void*)stream);
  if (err != 0) return fail(BCA_ERR_HIP, "counter kernel launch failed (hip error %d)", err);
  g_err.clear();
  return BCA_OK;
}

bca_status bca_attend_replayable(const bca_cache* c, int32_t layer, const bca_window_spec* s,
                                 int32_t* replayable) {
  if (!replayable) return fail(BCA_ERR_INVALID_ARG, "replayable is NULL");
  *replayable = 0;
  Plan p;
  bca_status st = make_plan(c, layer, s, c ? (c->d.kv_dtype == BCA_F32 ? BCA_F32 : BCA_BF16)
                                            : BCA_BF16, p);
  if (st != BCA_OK) return st;
  // Every ring slot holds one of the chunks t-S .. t-1 (so all S are visible
  // and consecutive appends keep them so), the window covers the whole ring,
  // and a requested reference is present: then the plan of chunk t is the
  // plan of every later chunk of a consecutive stream.
  const int S = c->d.ring_slots;
  const int64_t t = s->q_chunk_id;
  bool ok = s->history >= S && (!s->use_ref || c->ref_valid[layer]);
  for (int sl = 0; ok && sl < S; ++sl) {
    const int64_t id = c->slot[(size_t)layer * S + sl];
    // an empty slot (-1) never qualifies, also when t < S makes t - S negative
    ok = id >= 0 && id >= t - S && id <= t - 1;
  }
  *replayable = ok ? 1 : 0;
  g_err.clear();
  return BCA_OK;
}

bca_status bca_append_chunk(bca_cache* c, int32_t layer, int64_t chunk_id, int32_t is_ref,
                            const void* k, const void* v, int32_t in_dtype,
                            bca_stream_t stream) {
  return append_impl(c, layer, chunk_id, is_ref, k, v, in_dtype, stream, nullptr);
}

bca_status bca_append_chunk_rope(bca_cache* c, int32_t layer, int64_t chunk_id, int32_t is_ref,
                                 const void* k, const void* v, int32_t in_dtype,
                                 double rope_base, int64_t pos0, bca_stream_t stream) {
  bca_status st = check_rope(rope_base, pos0);
  if (st != BCA_OK) return st;
  const RopeArg r{std::log2(rope_base), pos0};
  return append_impl(c, layer, chunk_id, is_ref, k, v, in_dtype, stream, &r);
}

size_t bca_attend_workspace_bytes(const bca_cache* c, const bca_window_spec* s) {
  if (!c || !s) return 0;
  const int S = c->d.ring_slots, n = c->d.chunk_tokens;
  if (s->history < 0 || s->history > S || s->num_segments < 0 || s->num_segments > kMaxSegments)
    return 0;
  // The qkv dtype follows from the cache dtype (F32 -> F32, otherwise BF16).
  const int32_t qkv = c->d.kv_dtype == BCA_F32 ? BCA_F32 : BCA_BF16;
  const Kern k = kernel_for(qkv, c->d.kv_dtype);
  const TileShape ts = tile_shape(k);
  const int64_t q_tiles = (n + ts.bm - 1) / ts.bm;
  const int64_t units = (int64_t)c->d.num_heads * q_tiles;
  // Bound over every ring occupancy: 1 visible block (the current chunk) up to
  // all ring slots, the reference and the current chunk.
  size_t worst = 0;
  const int max_blocks = S + c->d.has_ref + 1;
  const bool blk = is_blk(c->d.kv_dtype);
  for (int blocks = 1; blocks <= max_blocks; ++blocks) {
    const int64_t cache_keys = blk ? (int64_t)(blocks - 1) * block_tiles(c->d) * 64
                                   : (int64_t)(blocks - 1) * n;
    int64_t T = (cache_keys + ts.bn - 1) / ts.bn + (n + ts.bn - 1) / ts.bn;
    int64_t P = choose_wgs(c, k, units, T, s->num_segments);
    if (pieces_bound(units, T, P) > 1)
      worst = std::max(worst, partial_bytes(P, slots_per_wg(units, P), ts.bm, c->d.head_dim));
  }
  if (k == Kern::FP8) worst += fp8_stage_bytes(c->d);
  if (blk) worst += cur_scale_bytes(c->d);
  return worst;
}

}  // extern "C"

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace for the rotated copies of Q and K of the current chunk.
size_t rope_stage_bytes(const bca_cache_desc& d, int32_t qkv_dtype) {
  return 2 * align256((size_t)d.chunk_tokens * d.num_heads * d.head_dim * elem_size(qkv_dtype));
}

bca_status attend_impl(const bca_cache* c, int32_t layer, const bca_window_spec* s,
                       const void* q, const void* k_cur, const void* v_cur, int32_t qkv_dtype,
                       void* o, float* lse, void* workspace, size_t workspace_bytes,
                       bca_stream_t stream, const RopeArg* rope, const int64_t* dev_t = nullptr) {
  Plan p;
  bca_status st = make_plan(c, layer, s, qkv_dtype, p);
  if (st != BCA_OK) return st;
  if (dev_t) {
    // the chunk id comes from the device: the bf16 and 8-bit ring paths, with
    // a ring that holds the S chunks before spec->q_chunk_id (then every later
    // chunk of a consecutive stream sees W blocks, in slots the kernel derives)
    if (c->d.kv_dtype == BCA_F32)
      return fail(BCA_ERR_UNSUPPORTED, "device-side chunk ids need a 16- or 8-bit cache");
    if (!aligned(dev_t, 8))
      return fail(BCA_ERR_INVALID_ARG, "d_q_chunk_id must be 8-byte aligned");
    const int S = c->d.ring_slots;
    for (int sl = 0; sl < S; ++sl) {
      const int64_t id = c->slot[(size_t)layer * S + sl];
      // empty slots (-1) are refused too: with t < S, t - S is negative
      if (id < 0 || id < s->q_chunk_id - S || id > s->q_chunk_id - 1)
        return fail(BCA_ERR_INVALID_ARG,
                    "ring slot %d holds chunk %lld, not one of the %d chunks before %lld", sl,
                    (long long)id, S, (long long)s->q_chunk_id);
    }
    if (s->use_ref && !c->ref_valid[layer])
      return fail(BCA_ERR_INVALID_ARG, "use_ref set but no reference chunk was appended");
    p.devt = 1;
  }
  if (!q || !k_cur || !v_cur || !o)
    return fail(BCA_ERR_INVALID_ARG, "q, k_cur, v_cur and o must not be NULL");
  if (!aligned(q, 16) || !aligned(k_cur, 16) || !aligned(v_cur, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)))
    return fail(BCA_ERR_INVALID_ARG, "q, k_cur, v_cur and o must be 16-byte aligned");
  const bca_cache_desc& d = c->d;
  // the rotated copies of Q and K follow the plan's own workspace regions
  const size_t rope_off = align256(p.ws_bytes);
  const size_t need = rope ? rope_off + rope_stage_bytes(d, qkv_dtype) : p.ws_bytes;
  if (need > 0) {
    if (!workspace) return fail(BCA_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if (!aligned(workspace, 256))
      return fail(BCA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(BCA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes,
                  need);
  }
  if (rope) {
    RopeStageArgs r;
    std::memset(&r, 0, sizeof r);
    char* qr = static_cast<char*>(workspace) + rope_off;
    char* kr = qr + rope_stage_bytes(d, qkv_dtype) / 2;
    r.src[0] = q;
    r.src[1] = k_cur;
    r.dst[0] = qr;
    r.dst[1] = kr;
    r.n = d.chunk_tokens;
    r.H = d.num_heads;
    r.log2_base = rope->log2_base;
    r.pos0 = rope->pos0;
    int err = launch_rope_stage((bca_dtype)qkv_dtype, d.head_dim, r, (void*)stream);
    if (err != 0) return fail(BCA_ERR_HIP, "rotary staging launch failed (hip error %d)", err);
    q = qr;
    k_cur = kr;
  }
  AttnArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = q;
  a.kcur = k_cur;
  a.vcur = v_cur;
  if (p.kern == Kern::FP8) {
    a.kcur_in = k_cur;
    a.vcur_in = v_cur;
    char* stage = static_cast<char*>(workspace) + p.stage_off;
    a.kcur = stage;
    a.vcur = stage + fp8_stage_bytes(d) / 2;
  }
  char* layer_k = c->mem + 2 * (size_t)layer * half_layer_bytes(d);
  a.kc = layer_k;
  a.vc = layer_k + half_layer_bytes(d);
  a.o = o;
  a.lse = lse;
  if (p.merge) {
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          part_o_bytes(p.wgs, p.spw, p.bm, d.head_dim));
    a.part_exp = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                            part_exp_offset(p.wgs, p.spw, p.bm, d.head_dim));
  }
  a.cache_head_elems = (int64_t)(d.ring_slots + d.has_ref) * d.chunk_tokens * d.head_dim;
  a.cache_span_elems = a.cache_head_elems;
  a.cache_row_elems = d.head_dim;
  a.n = d.chunk_tokens;
  a.H = d.num_heads;
  a.nk_cache = p.nk_cache;
  a.cache_tiles = p.cache_tiles;
  a.T = p.kv_tiles;
  a.QT = p.q_tiles;
  a.units = p.units;
  a.P = p.wgs;
  a.spw = p.spw;
  a.scale = s->scale;
  a.scale_log2 = (float)((double)s->scale * 1.4426950408889634);
  a.xcd_remap = (p.wgs % 8 == 0) ? 1 : 0;
  a.upc = p.units;  // one chunk
  if (p.devt) {
    a.dev_t = dev_t;
    a.dev_W = s->history;
    a.dev_S = d.ring_slots;
    a.dev_ref = s->use_ref ? 1 : 0;
  }
  a.nruns = p.nruns;
  for (int i = 0; i < p.nruns; ++i) a.runs[i] = p.runs[i];
  if (d.kv_dtype == BCA_FP8_E4M3)
    for (int h = 0; h < d.num_heads; ++h) {
      a.k_scale[h] = c->k_scale[(size_t)layer * d.num_heads + h];
      a.v_scale[h] = c->v_scale[(size_t)layer * d.num_heads + h];
    }
  if (p.blk) {
    a.blk = 1;
    a.i8k = p.i8k;
    a.tpb = p.tpb;
    a.nvis_cache = p.nvis - 1;
    a.ksc = block_scales(c, layer, 0);
    a.vsc = block_scales(c, layer, 1);
    a.cur_sc = reinterpret_cast<const float*>(static_cast<char*>(workspace) + p.stage_off +
                                              fp8_stage_bytes(d));
    for (int i = 0; i + 1 < p.nvis; ++i) a.vis_blk[i] = (int8_t)p.vis_block[i];
  }
  int err = launch_attention(p, a, d.head_dim, (void*)stream);
  if (err == -1) return fail(BCA_ERR_UNSUPPORTED, "no attention kernel for this dtype pair yet");
  if (err != 0) return fail(BCA_ERR_HIP, "attention launch failed (hip error %d)", err);
  g_err.clear();
  return BCA_OK;
}

// ---------------------------------------------------------------------------
// Training form: every chunk of a sequence at once (bca_attend_sequence).

bool seq_spec_ok(const bca_sequence_spec* s, int32_t qkv_dtype, std::string* why) {
  if (!s) return *why = "spec is NULL", false;
  if (s->num_heads <= 0 || s->chunk_tokens <= 0 || s->num_chunks <= 0)
    return *why = "num_heads, chunk_tokens and num_chunks must be > 0", false;
  if (s->prefix_tokens < 0) return *why = "prefix_tokens must be >= 0", false;
  if (s->history < 0) return *why = "history must be >= 0", false;
  if (s->num_segments < 0 || s->num_segments > kMaxSegments)
    return *why = "num_segments must be in [0, 64]", false;
  if (!std::isfinite(s->scale)) return *why = "scale must be finite", false;
  if (s->head_dim != 64 && s->head_dim != 128) return *why = "head_dim must be 64 or 128", false;
  if (qkv_dtype != BCA_F32 && qkv_dtype != BCA_BF16)
    return *why = "qkv_dtype must be BCA_F32 or BCA_BF16", false;
  // every byte offset into one head's K/V span must fit the kernels' 32-bit
  // buffer offsets
  const int64_t rows = (int64_t)s->prefix_tokens + (int64_t)s->num_chunks * s->chunk_tokens;
  const int64_t span = ((rows - 1) * s->num_heads * s->head_dim + s->head_dim) *
                       (int64_t)elem_size(qkv_dtype);
  if (rows > INT32_MAX / 2 || span > (int64_t)INT32_MAX - 4096)
    return *why = "K/V span per head exceeds 2 GiB", false;
  return true;
}

// Plan of chunks c .. c + count - 1, one launch. Their visible cache keys are
// the prefix and the window's earlier chunks, rows of the token-major K/V:
// one run when the two touch (c <= W), two otherwise. Chunks share a launch
// only when they see the same number of keys and the prefix (which stays) is
// a run of its own: then only the window's run moves, n rows per chunk.
void seq_plan(const bca_sequence_spec* s, int32_t qkv_dtype, int cus, int64_t c, int64_t count,
              Plan& p) {
  std::memset(&p, 0, sizeof p);
  const int64_t n = s->chunk_tokens, P = s->prefix_tokens;
  const int64_t first = std::max<int64_t>(0, c - s->history);  // first chunk of the window
  const int64_t hist = (c - first) * n;                        // window keys before chunk c
  p.nruns = 0;
  if (P > 0) p.runs[p.nruns++] = Run{0, (int32_t)P, 0, 0};
  if (hist > 0) {
    const int64_t phys = P + first * n;
    if (p.nruns > 0 && p.runs[0].phys + p.runs[0].len == phys)
      p.runs[0].len += (int32_t)hist;
    else
      p.runs[p.nruns++] = Run{(int32_t)P, (int32_t)hist, (int32_t)phys, 1};
  }
  p.nk_cache = (int32_t)(P + hist);
  p.kern = qkv_dtype == BCA_F32 ? Kern::F32 : Kern::BF16;
  p.seq = 1;
  const TileShape ts = tile_shape(p.kern);
  p.bm = ts.bm;
  p.bn = ts.bn;
  p.q_tiles = (int32_t)((n + p.bm - 1) / p.bm);
  p.cache_tiles = (p.nk_cache + p.bn - 1) / p.bn;
  p.kv_tiles = p.cache_tiles + (int32_t)((n + p.bn - 1) / p.bn);
  p.nk = p.nk_cache + (int32_t)n;
  p.units = (int32_t)(count * s->num_heads * p.q_tiles);
  p.wgs = (int32_t)choose_wgs_on(cus, p.kern, p.units, p.kv_tiles, s->num_segments);
  p.jmax = pieces_bound(p.units, p.kv_tiles, p.wgs);
  p.merge = p.jmax > 1 ? 1 : 0;
  p.spw = slots_per_wg(p.units, p.wgs);
  p.ws_bytes = p.merge ? partial_bytes(p.wgs, p.spw, p.bm, s->head_dim) : 0;
}

// The launches of a sequence. Chunks before the steady window go one by one;
// from chunk W (W + 1 with a prefix, where chunk W's window still touches
// the prefix) on every chunk sees the same number of keys, and the bf16
// kernel takes them all in one launch. The fp32 kernel runs chunk by chunk.
// With the automatic split on the bf16 path, when the chunks fill the device
// with units, the last kMaxGroups of those launches become one launch of
// groups (UnitGroup): that launch is cut stream-K style anyway, and the
// chunks before the window is full no longer pay a launch, a split and a
// merge each.
struct SeqLaunch {
  int64_t c, count;            // chunks c .. c + count - 1
  int32_t ng;                  // > 0: a launch of ng groups
  int64_t gc[kMaxGroups];      // first chunk of each group
  int64_t gn[kMaxGroups];      // chunks of each group
};

std::vector<SeqLaunch> seq_launches(const bca_sequence_spec* s, int32_t qkv_dtype, int cus) {
  const int64_t C = s->num_chunks;
  const int64_t steady = (int64_t)s->history + (s->prefix_tokens > 0 ? 1 : 0);
  const int64_t single = qkv_dtype == BCA_BF16 ? std::min(C, steady) : C;
  std::vector<std::pair<int64_t, int64_t>> plain;
  for (int64_t c = 0; c < single; ++c) plain.push_back({c, 1});
  if (single < C) plain.push_back({single, C - single});
  const size_t first = plain.size() > (size_t)kMaxGroups ? plain.size() - kMaxGroups : 0;
  const int64_t bm = tile_shape(Kern::BF16).bm;
  const int64_t units = (C - plain[first].first) * s->num_heads * ((s->chunk_tokens + bm - 1) / bm);
  const bool group = qkv_dtype == BCA_BF16 && s->num_segments == 0 && plain.size() - first >= 2 &&
                     units >= (int64_t)cus * wgs_per_cu(Kern::BF16);
  std::vector<SeqLaunch> out;
  const size_t ungrouped = group ? first : plain.size();
  for (size_t i = 0; i < ungrouped; ++i) {
    SeqLaunch L{};
    L.c = plain[i].first;
    L.count = plain[i].second;
    out.push_back(L);
  }
  if (group) {
    SeqLaunch L{};
    L.c = plain[first].first;
    L.count = C - L.c;
    L.ng = (int32_t)(plain.size() - first);
    for (int g = 0; g < L.ng; ++g) {
      L.gc[g] = plain[first + g].first;
      L.gn[g] = plain[first + g].second;
    }
    out.push_back(L);
  }
  return out;
}

// Plan of one launch of a sequence: seq_plan's, or for a launch of groups
// each group's own (its chunks' runs, keys and tiles), the units numbered
// group after group, and one range of tile iterations per resident work
// group over all of them.
void seq_launch_plan(const bca_sequence_spec* s, int32_t qkv_dtype, int cus, const SeqLaunch& L,
                     Plan& p) {
  if (L.ng == 0) {
    seq_plan(s, qkv_dtype, cus, L.c, L.count, p);
    return;
  }
  Plan gp;
  seq_plan(s, qkv_dtype, cus, L.gc[L.ng - 1], L.gn[L.ng - 1], gp);
  p = gp;  // the last group's fields stand as the launch's own
  int64_t units = 0, iters = 0;
  int nruns = 0;
  for (int g = 0; g < L.ng; ++g) {
    seq_plan(s, qkv_dtype, cus, L.gc[g], L.gn[g], gp);
    UnitGroup& G = p.grp[g];
    G = UnitGroup{};
    G.iter0 = iters;
    G.units0 = (int32_t)units;
    G.T = gp.kv_tiles;
    G.cache_tiles = gp.cache_tiles;
    G.nk_cache = gp.nk_cache;
    G.run0 = nruns;
    G.nruns = gp.nruns;
    G.chunk0 = (int32_t)(L.gc[g] - L.c);
    for (int i = 0; i < gp.nruns; ++i) p.runs[nruns++] = gp.runs[i];
    units += gp.units;
    iters += (int64_t)gp.units * gp.kv_tiles;
  }
  p.ngroups = L.ng;
  p.iters = iters;
  p.nruns = nruns;
  p.units = (int32_t)units;
  p.wgs = (int32_t)fewest_split_wgs(iters, units, (int64_t)cus * wgs_per_cu(p.kern),
                                     [&p, &L, units](int64_t u) -> int64_t {
                                       int g = 0;
                                       for (int i = 1; i < L.ng; ++i)
                                         if (u >= p.grp[i].units0) g = i;
                                       return p.grp[g].iter0 + (u - p.grp[g].units0) * p.grp[g].T;
                                     });
  int32_t worst = 1;
  for (int g = 0; g < L.ng; ++g) {
    const UnitGroup& G = p.grp[g];
    const int64_t gu = (g + 1 < L.ng ? p.grp[g + 1].units0 : units) - G.units0;
    for (int64_t u = 0; u < gu; ++u) {
      const int64_t x = G.iter0 + u * G.T;
      const int64_t pieces = first_wg(x + G.T - 1, iters, p.wgs) - first_wg(x, iters, p.wgs) + 1;
      worst = std::max<int32_t>(worst, (int32_t)pieces);
    }
  }
  p.jmax = worst;
  p.merge = worst > 1 ? 1 : 0;
  p.spw = 2;  // ranges end one unit and start the next
  p.ws_bytes = p.merge ? partial_bytes(p.wgs, p.spw, p.bm, s->head_dim) : 0;
}

// The workspace is the largest any launch of the sequence needs.
size_t seq_workspace(const bca_sequence_spec* s, int32_t qkv_dtype, int cus) {
  size_t ws = 0;
  for (const auto& l : seq_launches(s, qkv_dtype, cus)) {
    Plan p;
    seq_launch_plan(s, qkv_dtype, cus, l, p);
    ws = std::max(ws, p.ws_bytes);
  }
  return ws;
}

int seq_cus() {
  const int cus = device_compute_units();
  return cus > 0 ? cus : 256;
}

bca_status attend_sequence_impl(const bca_sequence_spec* s, const void* q, const void* k,
                                const void* v, int32_t qkv_dtype, void* o, float* lse,
                                void* workspace, size_t workspace_bytes, bca_stream_t stream) {
  std::string why;
  if (!s) return fail(BCA_ERR_INVALID_ARG, "spec is NULL");
  if (elem_size(qkv_dtype) == 0) return fail(BCA_ERR_INVALID_ARG, "qkv_dtype is not a bca_dtype");
  if ((qkv_dtype != BCA_F32 && qkv_dtype != BCA_BF16) ||
      (s->head_dim != 64 && s->head_dim != 128))
    return fail(BCA_ERR_UNSUPPORTED,
                "sequence attention runs F32 or BF16 with head_dim 64 or 128");
  if (!seq_spec_ok(s, qkv_dtype, &why)) return fail(BCA_ERR_INVALID_ARG, "%s", why.c_str());
  if (!q || !k || !v || !o) return fail(BCA_ERR_INVALID_ARG, "q, k, v and o must not be NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)))
    return fail(BCA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned (lse 4)");
  const int cus = seq_cus();
  const size_t need = seq_workspace(s, qkv_dtype, cus);
  if (need > 0) {
    if (!workspace) return fail(BCA_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if (!aligned(workspace, 256))
      return fail(BCA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(BCA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes,
                  need);
  }
  const int64_t n = s->chunk_tokens, H = s->num_heads, D = s->head_dim, P = s->prefix_tokens;
  const size_t es = elem_size(qkv_dtype);
  const int64_t rows = P + (int64_t)s->num_chunks * n;
  for (const auto& l : seq_launches(s, qkv_dtype, cus)) {
    const int64_t c = l.c;
    Plan p;
    seq_launch_plan(s, qkv_dtype, cus, l, p);
    AttnArgs a;
    std::memset(&a, 0, sizeof a);
    const size_t chunk_off = (size_t)(c * n * H * D) * es;      // chunk c's rows of q and o
    const size_t cur_off = (size_t)((P + c * n) * H * D) * es;  // chunk c's rows of k and v
    a.q = static_cast<const char*>(q) + chunk_off;
    a.kcur = static_cast<const char*>(k) + cur_off;
    a.vcur = static_cast<const char*>(v) + cur_off;
    a.kc = k;
    a.vc = v;
    a.o = static_cast<char*>(o) + chunk_off;
    a.lse = lse ? lse + (size_t)(c * H * n) : nullptr;
    if (p.merge) {
      a.part_o = static_cast<float*>(workspace);
      a.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                            part_o_bytes(p.wgs, p.spw, p.bm, (int)D));
      a.part_exp = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                              part_exp_offset(p.wgs, p.spw, p.bm, (int)D));
    }
    // the "cache" is the token-major K/V itself: heads d apart, rows H*d apart
    a.cache_head_elems = D;
    a.cache_span_elems = (rows - 1) * H * D + D;
    a.cache_row_elems = (int32_t)(H * D);
    a.n = (int32_t)n;
    a.H = (int32_t)H;
    a.nk_cache = p.nk_cache;
    a.cache_tiles = p.cache_tiles;
    a.T = p.kv_tiles;
    a.QT = p.q_tiles;
    a.units = p.units;
    a.P = p.wgs;
    a.spw = p.spw;
    a.scale = s->scale;
    a.scale_log2 = (float)((double)s->scale * 1.4426950408889634);
    a.xcd_remap = (p.wgs % 8 == 0) ? 1 : 0;
    // chunks c .. c + count - 1: unit u belongs to chunk c + u / upc
    a.upc = (int32_t)(H * p.q_tiles);
    a.chunk_rows = (int32_t)n;
    a.chunk_elems = n * H * D;
    a.chunk_lse = H * n;
    a.nruns = p.nruns;
    for (int i = 0; i < p.nruns; ++i) a.runs[i] = p.runs[i];
    a.ngroups = p.ngroups;
    a.iters = p.iters;
    for (int g = 0; g < p.ngroups; ++g) a.grp[g] = p.grp[g];
    const int err = launch_attention(p, a, (int)D, (void*)stream);
    if (err != 0)
      return fail(BCA_ERR_HIP, "attention launch for chunk %lld failed (hip error %d)",
                  (long long)c, err);
  }
  g_err.clear();
  return BCA_OK;
}

}  // namespace

extern "C" {

bca_status bca_attend(const bca_cache* c, int32_t layer, const bca_window_spec* s,
                      const void* q, const void* k_cur, const void* v_cur, int32_t qkv_dtype,
                      void* o, float* lse, void* workspace, size_t workspace_bytes,
                      bca_stream_t stream) {
  return attend_impl(c, layer, s, q, k_cur, v_cur, qkv_dtype, o, lse, workspace,
                     workspace_bytes, stream, nullptr);
}

bca_status bca_attend_noalloc(const bca_cache* c, int32_t layer, const bca_window_spec* s,
                              const void* q, const void* k_cur, const void* v_cur,
                              int32_t qkv_dtype, void* o, float* lse, bca_stream_t stream) {
  Plan p;
  bca_status st = make_plan(c, layer, s, qkv_dtype, p);
  if (st != BCA_OK) return st;
  if (p.ws_bytes > (size_t)BCA_NOALLOC_SCRATCH_BYTES)
    return fail(BCA_ERR_WORKSPACE,
                "bca_attend_noalloc: this call needs %zu bytes of scratch, more than the "
                "library's %zu (use bca_attend with a workspace)",
                p.ws_bytes, (size_t)BCA_NOALLOC_SCRATCH_BYTES);
  void* scratch = nullptr;
  if (p.ws_bytes > 0) {
    const int err = noalloc_scratch(&scratch);
    if (err != 0) return fail(BCA_ERR_HIP, "scratch address lookup failed (hip error %d)", err);
  }
  return attend_impl(c, layer, s, q, k_cur, v_cur, qkv_dtype, o, lse, scratch,
                     p.ws_bytes > 0 ? (size_t)BCA_NOALLOC_SCRATCH_BYTES : 0, stream, nullptr);
}

bca_status bca_attend_dev(const bca_cache* c, int32_t layer, const bca_window_spec* s,
                          const int64_t* d_q_chunk_id, const void* q, const void* k_cur,
                          const void* v_cur, int32_t qkv_dtype, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, bca_stream_t stream) {
  if (!d_q_chunk_id) return fail(BCA_ERR_INVALID_ARG, "d_q_chunk_id is NULL");
  return attend_impl(c, layer, s, q, k_cur, v_cur, qkv_dtype, o, lse, workspace,
                     workspace_bytes, stream, nullptr, d_q_chunk_id);
}

size_t bca_attend_rope_workspace_bytes(const bca_cache* c, const bca_window_spec* s) {
  if (!c || !s) return 0;
  const int32_t qkv = c->d.kv_dtype == BCA_F32 ? BCA_F32 : BCA_BF16;
  return align256(bca_attend_workspace_bytes(c, s)) + rope_stage_bytes(c->d, qkv);
}

bca_status bca_attend_rope(const bca_cache* c, int32_t layer, const bca_window_spec* s,
                           const void* q, const void* k_cur, const void* v_cur,
                           int32_t qkv_dtype, double rope_base, int64_t pos0, void* o,
                           float* lse, void* workspace, size_t workspace_bytes,
                           bca_stream_t stream) {
  bca_status st = check_rope(rope_base, pos0);
  if (st != BCA_OK) return st;
  const RopeArg r{std::log2(rope_base), pos0};
  return attend_impl(c, layer, s, q, k_cur, v_cur, qkv_dtype, o, lse, workspace,
                     workspace_bytes, stream, &r);
}

size_t bca_attend_sequence_workspace_bytes(const bca_sequence_spec* s, int32_t qkv_dtype) {
  std::string why;
  if (!seq_spec_ok(s, qkv_dtype, &why)) return 0;
  return seq_workspace(s, qkv_dtype, seq_cus());
}

bca_status bca_attend_sequence(const bca_sequence_spec* s, const void* q, const void* k,
                               const void* v, int32_t qkv_dtype, void* o, float* lse,
                               void* workspace, size_t workspace_bytes, bca_stream_t stream) {
  return attend_sequence_impl(s, q, k, v, qkv_dtype, o, lse, workspace, workspace_bytes, stream);
}

bca_status bca_cache_slot_chunk(const bca_cache* c, int32_t layer, int32_t slot,
                                int64_t* chunk_id) {
  if (!c || !chunk_id) return fail(BCA_ERR_INVALID_ARG, "cache or chunk_id is NULL");
  if (!layer_ok(c, layer)) return fail(BCA_ERR_INVALID_ARG, "layer %d out of range", layer);
  const int S = c->d.ring_slots;
  if (slot == S && c->d.has_ref) {
    *chunk_id = c->ref_valid[layer] ? c->ref_id[layer] : -1;
    return BCA_OK;
  }
  if (slot < 0 || slot >= S) return fail(BCA_ERR_INVALID_ARG, "slot %d out of range", slot);
  *chunk_id = c->slot[(size_t)layer * S + slot];
  return BCA_OK;
}

bca_status bca_cache_set_slot_chunk(bca_cache* c, int32_t layer, int32_t slot,
                                    int64_t chunk_id) {
  if (!c) return fail(BCA_ERR_INVALID_ARG, "cache is NULL");
  if (!layer_ok(c, layer)) return fail(BCA_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (chunk_id < -1) return fail(BCA_ERR_INVALID_ARG, "chunk_id must be >= -1");
  const int S = c->d.ring_slots;
  if (slot == S && c->d.has_ref) {
    c->ref_valid[layer] = chunk_id >= 0 ? 1 : 0;
    c->ref_id[layer] = chunk_id;
    return BCA_OK;
  }
  if (slot < 0 || slot >= S) return fail(BCA_ERR_INVALID_ARG, "slot %d out of range", slot);
  if (chunk_id >= 0 && chunk_id % S != slot)
    return fail(BCA_ERR_INVALID_ARG, "chunk %lld belongs in slot %lld, not %d",
                (long long)chunk_id, (long long)(chunk_id % S), slot);
  c->slot[(size_t)layer * S + slot] = chunk_id;
  int64_t nw = -1;
  for (int sl = 0; sl < S; ++sl) nw = std::max(nw, c->slot[(size_t)layer * S + sl]);
  c->newest[layer] = nw;
  return BCA_OK;
}

bca_status bca_attend_plan(const bca_cache* c, int32_t layer, const bca_window_spec* s,
                           bca_plan_info* out) {
  if (!out) return fail(BCA_ERR_INVALID_ARG, "out is NULL");
  if (!c) return fail(BCA_ERR_INVALID_ARG, "cache is NULL");
  Plan p;
  int32_t qkv = c->d.kv_dtype == BCA_F32 ? BCA_F32 : BCA_BF16;
  bca_status st = make_plan(c, layer, s, qkv, p);
  if (st != BCA_OK) return st;
  std::memset(out, 0, sizeof *out);
  out->num_visible_blocks = p.nvis;
  for (int i = 0; i < p.nvis; ++i) {
    out->visible_blocks[i] = p.vis_block[i];
    out->visible_chunk_ids[i] = p.vis_id[i];
  }
  out->visible_keys = p.nk;
  out->q_tiles = p.q_tiles;
  out->kv_tiles = p.kv_tiles;
  out->units = p.units;
  out->workgroups = p.wgs;
  out->max_pieces = p.jmax;
  out->merge = p.merge;
  out->workspace_bytes = p.ws_bytes;
  g_err.clear();
  return BCA_OK;
}

const char* bca_status_string(bca_status s) {
  switch (s) {
    case BCA_OK: return "BCA_OK";
    case BCA_ERR_INVALID_ARG: return "BCA_ERR_INVALID_ARG";
    case BCA_ERR_OUT_OF_ORDER: return "BCA_ERR_OUT_OF_ORDER";
    case BCA_ERR_WORKSPACE: return "BCA_ERR_WORKSPACE";
    case BCA_ERR_UNSUPPORTED: return "BCA_ERR_UNSUPPORTED";
    case BCA_ERR_HIP: return "BCA_ERR_HIP";
  }
  return "BCA_ERR_UNKNOWN";
}

const char* bca_last_error(void) { return g_err.c_str(); }

}  // extern "C"
