// bca_kernels.hip — gfx950 kernels of block-causal ring-KV chunk attention.
//
//   attn_bf16_kernel   bf16 flash attention on MFMA (v_mfma_f32_32x32x16_bf16)
//   attn_fp8_kernel    8-bit-cache flash attention: e4m3 K and V on the fp8
//                      MFMA (v_mfma_f32_32x32x64_f8f6f4), or int8 K on the
//                      int8 MFMA (v_mfma_i32_32x32x32_i8) with e4m3 V
//   attn_f32_kernel    fp32 flash attention on the vector ALUs
//   merge_lanes_kernel log-sum-exp merge of segment partials (bf16, 8-bit paths)
//   merge_kernel       the same for the fp32 path's partials
//   append_copy_kernel fused K/V write of one chunk into its ring slot
//   append_amax_kernel per-head scales of a per-block 8-bit append
//   append_fp8_kernel  the same with 8-bit quantisation (also the 8-bit copy of
//                      the current chunk that the 8-bit kernels read)
//   rope_stage_kernel  rotary embedding of the current chunk's Q and K into
//                      staging copies
//   append_rope_k_kernel  the rotated K of an append (copy or 8-bit codes)
//   counter_advance_kernel  the device-side chunk counter of a replayed step
//   mfma_peak_kernel, mfma_peak_fp8_kernel  matrix-core rate probes
//
// What is computed follows "WanToFight" (xllm-io review), section 3 model
// components table (block-causal attention: bidirectional in the chunk, causal
// over a bounded window of chunks; rolling KV cache), and "Matrix-Game 4.0"
// (paper summary), prerequisite "causal autoregression and KV cache" (ring
// buffer overwritten in place; the window split into intervals merged by
// log-sum-exp) and "technical novelty". The pages' kernels were written for
// other GPUs; the tiling below is designed for CDNA4 wave64 MFMA and LDS.
//
// Work decomposition shared by the attention kernels. The keys a query chunk
// sees are the same for every row of the chunk (the mask is block-causal), so
// the host lists the visible keys as "runs" of consecutive rows and every
// (head, query tile) unit has the same number T of key tiles. The units*T tile
// iterations are cut into P consecutive, equal ranges, one per work group; a
// unit whose tiles span several ranges is computed as several segments, each
// written as a normalised partial output plus its LSE, and the merge kernel
// combines them. A unit computed whole writes the final output. (With P a
// multiple of the unit count every unit gets the same number of equal
// segments; otherwise ranges cross unit boundaries, "stream-K" style.) A
// sequence launch may hold groups of units of different lengths (UnitGroup),
// numbered group after group.
#include <hip/hip_runtime.h>

#include <mutex>

#include "bca_internal.h"
#include "../../include/bca_probe.h"

namespace bca {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ int64_t range_begin(int64_t w, int64_t I, int64_t P) {
  return w * I / P;
}

// First work group whose range contains iteration x.
__device__ __forceinline__ int64_t first_wg_of(int64_t x, int64_t I, int64_t P) {
  return ((x + 1) * P + I - 1) / I - 1;
}

// Partial-output slot of work group w's part of unit u (T tiles per unit).
// A range touches at most two units whose results stay partial: the one it
// starts in and the one it ends in, so each work group owns spw <= 2 slots
// (spw = 1 when every range lies within one unit) and the workspace is
// bounded by the launch's work groups, not by its units.
__device__ __forceinline__ int64_t part_slot(int64_t w, int64_t u, int64_t I, int64_t T,
                                             int64_t P, int spw) {
  return (int64_t)spw * w + (u != range_begin(w, I, P) / T ? 1 : 0);
}

// Launches whose units differ in length (ngroups > 0, see UnitGroup): the
// group holding unit u or iteration it, the launch's iterations, the first
// iteration of unit u, the unit holding iteration it. With ngroups = 0 every
// unit has T tiles.
template <typename Args>
__device__ __forceinline__ int group_of_unit(const Args& a, int64_t u) {
  int g = 0;
  for (int i = 1; i < a.ngroups; ++i)
    if (u >= a.grp[i].units0) g = i;
  return g;
}
template <typename Args>
__device__ __forceinline__ int group_of_iter(const Args& a, int64_t it) {
  int g = 0;
  for (int i = 1; i < a.ngroups; ++i)
    if (it >= a.grp[i].iter0) g = i;
  return g;
}
template <typename Args>
__device__ __forceinline__ int64_t total_iters(const Args& a) {
  return a.ngroups > 0 ? a.iters : (int64_t)a.units * a.T;
}
template <typename Args>
__device__ __forceinline__ int64_t unit_first_iter(const Args& a, int64_t u) {
  if (a.ngroups <= 0) return u * a.T;
  const UnitGroup& G = a.grp[group_of_unit(a, u)];
  return G.iter0 + (u - G.units0) * G.T;
}
template <typename Args>
__device__ __forceinline__ int64_t unit_of_iter(const Args& a, int64_t it) {
  if (a.ngroups <= 0) return it / a.T;
  const UnitGroup& G = a.grp[group_of_iter(a, it)];
  return G.units0 + (it - G.iter0) / G.T;
}
// part_slot for units of any length.
template <typename Args>
__device__ __forceinline__ int64_t part_slot_of(const Args& a, int64_t w, int64_t u, int64_t I) {
  return (int64_t)a.spw * w + (u != unit_of_iter(a, range_begin(w, I, a.P)) ? 1 : 0);
}

// Work-group ids are handed to the 8 XCDs round robin (id % 8). Remapping so
// that XCD x gets the contiguous range [x P/8, (x+1) P/8) keeps the work
// groups that read the same head's K/V on one XCD and its L2.
__device__ __forceinline__ int logical_wg(const AttnArgs& a) {
  int b = blockIdx.x;
  if (a.xcd_remap) {
    const int per = a.P >> 3;
    b = (b & 7) * per + (b >> 3);
  }
  return b;
}

// K/V rows are read with buffer loads. Each head has two resources per
// tensor: its cache matrix [(S+R)*n][d] and its rows of the current chunk
// (row stride H*d). An offset past a resource's size reads as zero, which
// is how rows beyond the last visible key become zero rows without a branch.
constexpr int kBufDword3 = 0x00020000;  // raw buffer, gfx9 family
constexpr int kOob = 0x7ffffff0;
// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt 0 and nothing else
constexpr int kVmcnt0 = 0x0F70;

struct HeadSrc {
  const char* cache;  // this head's cache matrix
  const char* cur;    // this head's first row of the current chunk
  int cache_bytes;
  int cur_bytes;
};

// A pointer every lane agrees on, held in scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ HeadSrc head_src(const void* cache_base, const void* cur_base,
                                            const AttnArgs& a, int h, int D, int es_cache,
                                            int es_cur) {
  HeadSrc r;
  r.cache = uniform_ptr(static_cast<const char*>(cache_base) +
                        (int64_t)h * a.cache_head_elems * es_cache);
  r.cache_bytes = (int)(a.cache_span_elems * es_cache);
  r.cur = uniform_ptr(static_cast<const char*>(cur_base) + (int64_t)h * D * es_cur);
  r.cur_bytes = (int)(((int64_t)(a.n - 1) * a.H * D + D) * es_cur);
  return r;
}

__device__ __forceinline__ uint4 buf16(const char* base, int bytes, int off) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(base), (short)0, bytes, kBufDword3);
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Loads 16 bytes at byte column `colb` of NR cache-key rows (key numbers j[i]
// in the cache part of the key order) of the tile of BN keys starting at j0;
// `ri` is the run holding j0. Keys at or beyond nk_cache read as zeros.
template <int NR, int BN>
__device__ __forceinline__ void load_cache_rows(const AttnArgs& a, const HeadSrc& src, int D,
                                                int es, int j0, int ri, const int (&j)[NR],
                                                int colb, uint4 (&out)[NR]) {
  const Run R0 = a.runs[ri];
  if (j0 + BN <= R0.vstart + R0.len) {
#pragma unroll
    for (int i = 0; i < NR; ++i)
      out[i] = buf16(src.cache, src.cache_bytes,
                     (R0.phys + j[i] - R0.vstart) * a.cache_row_elems * es + colb);
    return;
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) out[i] = make_uint4(0, 0, 0, 0);
  for (int r = ri; r < a.nruns; ++r) {
    const Run R = a.runs[r];
    if (R.vstart >= j0 + BN) break;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const bool in = j[i] >= R.vstart && j[i] < R.vstart + R.len;
      const uint4 v = buf16(src.cache, src.cache_bytes,
                            in ? (R.phys + j[i] - R.vstart) * a.cache_row_elems * es + colb
                               : kOob);
      out[i].x |= v.x;
      out[i].y |= v.y;
      out[i].z |= v.z;
      out[i].w |= v.w;
    }
  }
}

// Advances ri to the run holding key j0 (runs are visited in increasing order).
__device__ __forceinline__ int advance_run(const AttnArgs& a, int ri, int j0) {
  while (ri + 1 < a.nruns && a.runs[ri].vstart + a.runs[ri].len <= j0) ++ri;
  return ri;
}

// Max and sum over the lane pair l, l^32 (the two halves of a row's keys):
// v_permlane32_swap exchanges the upper half of one operand with the lower
// half of the other, so with both operands x every lane ends up holding x of
// itself and of its partner (in either order), which is all a max or a sum
// needs.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// The softmax's maxima propagate NaN (IEEE maximum, v_maximum3_f32): unlike
// fmaxf they need no quieting of the MFMA results first, and a NaN score makes
// its row NaN either way.
__device__ __forceinline__ float max3n(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
__device__ __forceinline__ float xhalf_maxn(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// bf16 attention on MFMA.
//
// Work group: 512 threads = 8 waves in two groups of 4. BM = 256 query rows:
// wave w of group g owns rows 128g + 32(w%4) .. +31. Key tiles of BN = 64 keys.
//
// Ping-pong: the groups run the same sequence -- QK(0) | SM(0) | PV(0)+QK(1) |
// SM(1) | PV(1)+QK(2) | ... -- one phase apart, with a work-group barrier
// between phases, so in every phase one group issues MFMAs (PV of one tile and
// QK of the next: 32 per wave) while the other runs the softmax on the vector
// ALUs of the same SIMDs. The MFMA group raises its wave priority for its
// phase. Every key tile in LDS serves all 256 rows.
//
// Tiles reach LDS by buffer loads with an LDS destination (lane L of a
// wave-wide 16-byte load lands at M0 + 16 L), four stages deep: tile r+2 is
// requested at the start of phase 2r and first read at phase 2r+4. K and V stay
// row-major; rows are XOR-swizzled at 16-byte granularity so both read
// patterns below are free of bank conflicts.
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
// (A = 32 keys x 16 dims from LDS, B = Q^T held in registers for the unit).
// In the 32x32 result lane l holds query l%32 and 16 keys, so a row's max and
// sum need one exchange with lane l^32. O^T += V^T P^T takes P^T from
// registers as the B operand, its k index running over keys in the order the
// score layout leaves them ({4h..4h+3, 8+4h..8+4h+3} of every 16 keys for
// lane half h); V^T comes from row-major V through ds_read_b64_tr_b16 (within
// each group of 16 lanes, source lane a+4k points at 4 consecutive dims of key
// key0+k, and result lane 4a+b receives those 4 keys at one dim).
//
// Online softmax in base 2 with a lazy rescale: the running maximum moves only
// when a tile exceeds it by more than 8 (a factor 256), so O and l are
// rescaled on few tiles.
template <int D>
struct Bf16Cfg {
  static constexpr int BM = 256, BN = 64, NT = 512, NW = 8, NSTAGE = 4;
  static constexpr int ROWB = D * 2;                  // bytes per key row
  static constexpr int CPR = D / 8;                   // 16-byte chunks per row
  static constexpr int TILE_BYTES = BN * ROWB;        // K (or V) of one tile
  static constexpr int STAGE = 2 * TILE_BYTES;        // K then V
  static constexpr int RPI = 1024 / ROWB;             // rows per wave-wide 16-byte load
  static constexpr int IPW = TILE_BYTES / 1024 / NW;  // such loads per wave per tensor
  static constexpr int LOADS = 2 * IPW;               // per wave per tile
};

// Physical 16-byte chunk of logical chunk c in tile row r is c ^ swizzle(r).
// K rows are read 16 at a time at one logical chunk: the swizzle spreads them
// over all 16 chunk slots of a 256-byte bank line. V is read 4 rows x 64 bytes
// per 32 lanes: the swizzle moves each of the 4 rows to a different 64-byte
// quarter of the bank line.
template <int D>
__device__ __forceinline__ int k_swizzle(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swizzle(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// One wave-wide 16-byte buffer load into LDS (lane L -> lds + 16 L).
// Issued through inline assembly on purpose: the kernels wait for these
// loads themselves (s_waitcnt vmcnt before the work-group barrier that
// precedes each use), and the compiler, which cannot tell which LDS stage a
// load writes, would otherwise wait for all of them before every LDS read.
// base must be wave-uniform (it becomes a scalar buffer resource).
__device__ __forceinline__ void lds_load16(const char* base, int bytes, int off,
                                           unsigned char* lds) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4_t rsrc;
  rsrc[0] = (int)__builtin_amdgcn_readfirstlane((uint32_t)p);
  rsrc[1] = (int)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xffffu);
  rsrc[2] = bytes;
  rsrc[3] = kBufDword3;
  const unsigned lds_addr = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)(lds));
  // m0 is reserved by the compiler: save it, point it at the LDS destination,
  // restore it.
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(rsrc), "s"(lds_addr)
      : "memory");
}

// Scalar state of the tile requests of one unit: the run that holds the next
// cache tile, kept in registers and reloaded only when a tile crosses into
// the next run.
struct FetchRun {
  int ri, vstart, vend, phys;
  int shift;  // rows a moving run is displaced by (the unit's chunk in a batched launch)
};

// A unit's own runs and cache tiles on the sequence path (those of its group
// in a launch of groups): runs[rb .. rb + rn), ct key tiles over cache keys.
struct UnitRuns {
  int rb, rn, ct;
};

// Runs of a launch whose visible slots the kernel derives itself
// (bca_attend_dev): built once per work group in LDS. A per-block cache has
// one run per visible block; dev_vis keeps that block's index (ring slot, or
// S for the reference) for its scales.
__shared__ Run dev_runs[kMaxBlocks];
__shared__ int dev_vis[kMaxBlocks];
__shared__ int dev_nruns;

template <bool DEVT>
__device__ __forceinline__ Run run_of(const AttnArgs& a, int ri) {
  if constexpr (DEVT) return dev_runs[ri];
  else return a.runs[ri];
}
template <bool DEVT>
__device__ __forceinline__ int nruns_of(const AttnArgs& a) {
  if constexpr (DEVT) return dev_nruns;
  else return a.nruns;
}

// The visible ring slots of query chunk t = *a.dev_t when the ring holds
// consecutive ids: chunks t-W .. t-1 sit in slots (t-W) mod S .. (t-1) mod S.
// The runs are built as the host builds them (ascending physical blocks, the
// reference block S last; adjacent blocks merged, or with BLK one run per
// block, each padded to a.tpb whole key tiles), so the launch computes
// exactly what a host-planned call for the same chunk computes.
template <bool BLK>
__device__ __forceinline__ void build_dev_runs(const AttnArgs& a) {
  const int64_t t = *a.dev_t;
  const int S = a.dev_S, W = a.dev_W, n = a.n;
  const int s0 = (int)((((t - W) % S) + S) % S);
  int nr = 0, nb = 0;
  auto add = [&](int b) {
    if (BLK) {
      dev_runs[nr] = Run{nb * a.tpb * 64, n, b * n, 0};
      dev_vis[nr] = b;
      ++nr;
    } else if (nr > 0 && dev_runs[nr - 1].phys + dev_runs[nr - 1].len == b * n) {
      dev_runs[nr - 1].len += n;
    } else {
      dev_runs[nr] = Run{nb * n, n, b * n, 0};
      ++nr;
    }
    ++nb;
  };
  const int wrap = s0 + W - S;  // slots 0 .. wrap-1 when the window wraps
  for (int b = 0; b < wrap; ++b) add(b);
  for (int b = s0; b < s0 + W && b < S; ++b) add(b);
  if (a.dev_ref) add(S);
  dev_nruns = nr;
}

template <bool DEVT = false>
__device__ __forceinline__ FetchRun fetch_run_at(const AttnArgs& a, int ri, int shift = 0) {
  const Run R = run_of<DEVT>(a, ri);
  FetchRun f;
  f.ri = ri;
  f.shift = shift;
  f.vstart = R.vstart;
  f.vend = f.vstart + R.len;
  f.phys = R.phys + (R.moves ? shift : 0);
  return f;
}
// Run ri of a unit whose runs start at runs[rb].
__device__ __forceinline__ FetchRun fetch_run_in(const AttnArgs& a, int rb, int ri, int shift) {
  const Run R = a.runs[rb + ri];
  FetchRun f;
  f.ri = ri;
  f.shift = shift;
  f.vstart = R.vstart;
  f.vend = f.vstart + R.len;
  f.phys = R.phys + (R.moves ? shift : 0);
  return f;
}

// Per-lane constants of the request pattern: the tile row each of the lane's
// IPW loads covers and its swizzled byte column for K and for V.
template <int D>
struct FetchLane {
  int r[Bf16Cfg<D>::IPW];
  int roff[Bf16Cfg<D>::IPW];  // r * cache row pitch in bytes
  int kcol[Bf16Cfg<D>::IPW];
  int vcol[Bf16Cfg<D>::IPW];
};

template <int D>
__device__ __forceinline__ FetchLane<D> fetch_lane(int wave, int lane, int rowb) {
  using C = Bf16Cfg<D>;
  FetchLane<D> f;
  const int lrow = lane / C::CPR, lchunk = lane % C::CPR;
#pragma unroll
  for (int q = 0; q < C::IPW; ++q) {
    const int r = (wave * C::IPW + q) * C::RPI + lrow;
    f.r[q] = r;
    f.roff[q] = r * rowb;
    f.kcol[q] = (lchunk ^ k_swizzle<D>(r)) << 4;
    f.vcol[q] = (lchunk ^ v_swizzle<D>(r)) << 4;
  }
  return f;
}

// Requests K and V of key tile `tile` into one LDS stage; completion is
// awaited with vmcnt before the work-group barrier that precedes its use.
// Wave w's load q fills the 1 KB of the stage at (w IPW + q) KB. SEQ: cache
// rows are a token-major sequence (row pitch a.cache_row_elems); otherwise
// the ring's head-major rows of d elements.
template <int D, bool SEQ, bool DEVT>
__device__ __forceinline__ void bf16_fetch_tile(const AttnArgs& a, const HeadSrc& ks,
                                                const HeadSrc& vs, int tile, FetchRun& fr,
                                                const FetchLane<D>& fl, unsigned char* stage,
                                                int wave, const UnitRuns& ur) {
  using C = Bf16Cfg<D>;
  unsigned char* kdst = stage + wave * C::IPW * 1024;
  unsigned char* vdst = kdst + C::TILE_BYTES;
  // the unit's runs and cache tiles: its own on the sequence path
  const int ct = SEQ ? ur.ct : a.cache_tiles;
  const int rn = SEQ ? ur.rn : nruns_of<DEVT>(a);
  const int rb = SEQ ? ur.rb : 0;
  if (tile < ct) {
    const int j0 = tile * C::BN;
    while (j0 >= fr.vend && fr.ri + 1 < rn)
      fr = SEQ ? fetch_run_in(a, rb, fr.ri + 1, fr.shift) : fetch_run_at<DEVT>(a, fr.ri + 1, fr.shift);
    const int rowb = SEQ ? a.cache_row_elems * 2 : C::ROWB;
    if (j0 + C::BN <= fr.vend) {
      // the whole tile lies in one run
      const int base = (fr.phys + j0 - fr.vstart) * rowb;
#pragma unroll
      for (int q = 0; q < C::IPW; ++q) {
        const int off = base + fl.roff[q];
        lds_load16(ks.cache, ks.cache_bytes, off + fl.kcol[q], kdst + q * 1024);
        lds_load16(vs.cache, vs.cache_bytes, off + fl.vcol[q], vdst + q * 1024);
      }
    } else {
      // the tile crosses run boundaries or ends in padding
#pragma unroll
      for (int q = 0; q < C::IPW; ++q) {
        const int j = j0 + fl.r[q];
        int phys = -1;
        for (int rr = fr.ri; rr < rn; ++rr) {
          const Run R = run_of<DEVT>(a, rb + rr);
          if (R.vstart >= j0 + C::BN) break;
          if (j >= R.vstart && j < R.vstart + R.len)
            phys = R.phys + (SEQ && R.moves ? fr.shift : 0) + j - R.vstart;
        }
        const int koff = phys >= 0 ? phys * rowb + fl.kcol[q] : kOob;
        const int voff = phys >= 0 ? phys * rowb + fl.vcol[q] : kOob;
        lds_load16(ks.cache, ks.cache_bytes, koff, kdst + q * 1024);
        lds_load16(vs.cache, vs.cache_bytes, voff, vdst + q * 1024);
      }
    }
  } else {
    const int r0 = (tile - ct) * C::BN;
#pragma unroll
    for (int q = 0; q < C::IPW; ++q) {
      const int row = r0 + fl.r[q];
      const int rowoff = row * a.H * C::ROWB;
      const int koff = row < a.n ? rowoff + fl.kcol[q] : kOob;
      const int voff = row < a.n ? rowoff + fl.vcol[q] : kOob;
      lds_load16(ks.cur, ks.cur_bytes, koff, kdst + q * 1024);
      lds_load16(vs.cur, vs.cur_bytes, voff, vdst + q * 1024);
    }
  }
}

// Keys of `tile` that are real (the rest of the tile is padding), for a
// unit with cache_tiles tiles over nk_cache cache keys and n keys of its own.
__device__ __forceinline__ int tile_valid_of(int cache_tiles, int nk_cache, int n, int tile,
                                             int bn) {
  if (tile < cache_tiles) return min(bn, nk_cache - tile * bn);
  return min(bn, n - (tile - cache_tiles) * bn);
}
__device__ __forceinline__ int tile_valid(const AttnArgs& a, int tile, int bn) {
  return tile_valid_of(a.cache_tiles, a.nk_cache, a.n, tile, bn);
}

// Work-group barrier without the memory fences __syncthreads() adds (those
// would wait for every outstanding tile fetch). LDS reads issued before it
// have all been consumed by MFMAs or waited for explicitly.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_barrier" ::: "memory");
}

// Per-wave state of one unit in the ping-pong kernel.
template <int D>
struct PPState {
  f32x16_t o[D / 32];  // O^T accumulator: dims 32db + 8(e/4) + 4hi + e%4, query l%32
  f32x16_t s[2];       // S^T of the tile (keys 0-31, 32-63) between its QK and its softmax
  bf16x8_t pf[4];      // P^T of the tile (16-key steps) between its softmax and its PV
  float m_run, l_run;  // running max (base 2, scaled) and this lane's partial sum
};

// One MFMA phase: PV of the tile in stage SV and/or QK of the tile in stage
// SK. The 16 PV and 16 QK MFMAs alternate; consecutive QK MFMAs go to the two
// independent 32-key score blocks, and the LDS operands are requested AHEAD
// steps before their use. sched_barrier keeps the compiler from sinking the
// requests next to their uses.
template <int D, bool PV, bool QK>
__device__ __forceinline__ void pp_gemm(PPState<D>& st, const unsigned char* SV,
                                        const unsigned char* SK, const int (&koff)[D / 16],
                                        const int (&voff)[D / 32],
                                        const bf16x8_t (&qf)[D / 16]) {
  using C = Bf16Cfg<D>;
  constexpr int NPV = PV ? 4 * (D / 32) : 0;  // PV MFMAs: (kk 0..3, db)
  constexpr int NQK = QK ? 2 * (D / 16) : 0;  // QK MFMAs: (kk, key block 0..1)
  constexpr int NSTEP = NPV > NQK ? NPV : NQK;
  constexpr int AHEAD = 3;
  bf16x8_t vf[NSTEP + AHEAD], kf[NSTEP + AHEAD];
  auto load_v = [&](int i) {
    if (i < NPV) {
      const int kk = i / (D / 32), db = i % (D / 32);
      const unsigned char* vp = SV + voff[db] + 16 * kk * C::ROWB;
      const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp));
      const bf16x4_t h4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp + 8 * C::ROWB));
      vf[i] = __builtin_shufflevector(lo, h4, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  auto load_k = [&](int i) {
    if (i < NQK) {
      const int kk = i >> 1, kb = i & 1;
      kf[i] = *reinterpret_cast<const bf16x8_t*>(SK + koff[kk] + kb * 32 * C::ROWB);
    }
  };
  f32x16_t acc0 = f32x16_t{}, acc1 = f32x16_t{};
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) {
    load_v(i);
    load_k(i);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NSTEP; ++i) {
    if (i < NPV) {
      const int db = i % (D / 32), kk = i / (D / 32);
      st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], st.pf[kk], st.o[db], 0, 0, 0);
    }
    if (i < NQK) {
      if (i & 1)
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i >> 1], acc1, 0, 0, 0);
      else
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i >> 1], acc0, 0, 0, 0);
    }
    load_v(i + AHEAD);
    load_k(i + AHEAD);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (QK) {
    st.s[0] = acc0;
    st.s[1] = acc1;
  }
}

// Online softmax of the tile's scores (lim = real keys of the tile).
template <int D>
__device__ __forceinline__ void pp_softmax(PPState<D>& st, int lim, int hi, float c) {
  if (lim < 64) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kr = 8 * (e >> 2) + 4 * hi + (e & 3);
      if (kr >= lim) st.s[0][e] = -INFINITY;
      if (32 + kr >= lim) st.s[1][e] = -INFINITY;
    }
  }
  // maximum over the 32 scores (a tree of 3-input maxima) and the partner lane
  const f32x16_t v0 = st.s[0], v1 = st.s[1];
  float m[11];
#pragma unroll
  for (int e = 0; e < 5; ++e) m[e] = max3n(v0[3 * e], v0[3 * e + 1], v0[3 * e + 2]);
#pragma unroll
  for (int e = 0; e < 5; ++e) m[5 + e] = max3n(v1[3 * e], v1[3 * e + 1], v1[3 * e + 2]);
  m[10] = __builtin_elementwise_maximum(v0[15], v1[15]);
  const float n0 = max3n(m[0], m[1], m[2]), n1 = max3n(m[3], m[4], m[5]);
  const float n2 = max3n(m[6], m[7], m[8]), n3 = __builtin_elementwise_maximum(m[9], m[10]);
  const float mx = xhalf_maxn(max3n(n0, n1, __builtin_elementwise_maximum(n2, n3)));
  const float mxs = mx * c;
  const bool need = !(mxs <= st.m_run + 8.0f);
  if (__any(need)) {
    const float m_new = fmaxf(st.m_run, mxs);
    const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.o[db] *= alpha;
    st.l_run *= alpha;
    st.m_run = m_new;
  }
  const float m_use = st.m_run == -INFINITY ? 0.f : st.m_run;
  f32x16_t p0, p1;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    p0[e] = __builtin_amdgcn_exp2f(fmaf(v0[e], c, -m_use));
    p1[e] = __builtin_amdgcn_exp2f(fmaf(v1[e], c, -m_use));
  }
  // sum as a tree (independent adds instead of one long chain)
  float t8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) t8[e] = (p0[e] + p0[e + 8]) + (p1[e] + p1[e + 8]);
  st.l_run += ((t8[0] + t8[4]) + (t8[1] + t8[5])) + ((t8[2] + t8[6]) + (t8[3] + t8[7]));
  st.pf[0] = __builtin_convertvector(p0.lo, bf16x8_t);
  st.pf[1] = __builtin_convertvector(p0.hi, bf16x8_t);
  st.pf[2] = __builtin_convertvector(p1.lo, bf16x8_t);
  st.pf[3] = __builtin_convertvector(p1.hi, bf16x8_t);
}

// SEQ: a launch of bca_attend_sequence (token-major cache rows, units of
// several chunks); otherwise a ring-cache call, where that generality would
// only cost scalar registers.
// DEVT: a bca_attend_dev launch; the work group derives the visible slots
// from the device-side chunk id first (build_dev_runs).
template <int D, bool SEQ, bool DEVT>
__global__ __launch_bounds__(512) void attn_bf16_kernel(const AttnArgs a) {
  using C = Bf16Cfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::NSTAGE * C::STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int w = logical_wg(a);
  const int64_t I = SEQ ? total_iters(a) : (int64_t)a.units * a.T;
  int64_t it = range_begin(w, I, a.P);
  const int64_t it_end = range_begin(w + 1, I, a.P);

  // LDS read offsets within a stage. K: row l32 (+32 for keys 32-63), logical
  // chunk 2kk + hi.
  int koff[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    koff[kk] = l32 * C::ROWB + (((2 * kk + hi) ^ k_swizzle<D>(l32)) << 4);
  // V (transposed reads): group g16 = lane/16, i = lane%16 = ai + 4k; rows
  // 4 hi + k of each 8-key step, dims 32 db + 16 (g16%2) + 4 ai .. +3.
  int voff[D / 32];
  {
    const int g16 = lane >> 4, i = lane & 15, ai = i & 3, k = i >> 2;
    const int c0 = 2 * (g16 & 1) + (ai >> 1);
    const int kx = D == 128 ? k : (k >> 1);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      voff[db] = C::TILE_BYTES + (4 * hi + k) * C::ROWB + ((4 * (db ^ kx) + c0) << 4) +
                 (ai & 1) * 8;
  }
  const FetchLane<D> fl = fetch_lane<D>(wave, lane, SEQ ? a.cache_row_elems * 2 : C::ROWB);
  if constexpr (DEVT) {
    if (tid == 0) build_dev_runs<false>(a);
    __syncthreads();
  }

  while (it < it_end) {
    // the unit holding iteration it: its length, first iteration and runs
    // (on the sequence path those of its group in a launch of groups)
    int u, t0, T;
    UnitRuns ur{0, 0, 0};
    int nkc = 0, shift = 0;
    if constexpr (SEQ) {
      T = a.T;
      ur = UnitRuns{0, a.nruns, a.cache_tiles};
      nkc = a.nk_cache;
      int64_t gi0 = 0;
      int gu0 = 0, gc0 = 0;
      if (a.ngroups > 0) {
        const UnitGroup& G = a.grp[group_of_iter(a, it)];
        T = G.T;
        ur = UnitRuns{G.run0, G.nruns, G.cache_tiles};
        nkc = G.nk_cache;
        gc0 = G.chunk0;
        gi0 = G.iter0;
        gu0 = G.units0;
      }
      u = gu0 + (int)((it - gi0) / T);
      t0 = (int)(it - gi0 - (int64_t)(u - gu0) * T);
      shift = (u / a.upc - gc0) * a.chunk_rows;
    } else {
      u = (int)(it / a.T);
      t0 = (int)(it - (int64_t)u * a.T);
      T = a.T;
    }
    const int t1 = (int)((it_end - it) < (int64_t)(T - t0) ? t0 + (it_end - it) : T);
    const int nt = t1 - t0;
    const int ci = SEQ ? __builtin_amdgcn_readfirstlane(u / a.upc) : 0;  // chunk of the launch
    const int ul = u - ci * a.upc;
    const int h = __builtin_amdgcn_readfirstlane(ul / a.QT);
    const int qt = ul - h * a.QT;
    const int q0 = qt * C::BM + (wave & 7) * 32;  // = 128 grp + 32 (wave % 4)
    const bool wave_rows = q0 < a.n;
    const int64_t cel = SEQ ? (int64_t)ci * a.chunk_elems : 0;  // the chunk's first q/k/v/o element
    const HeadSrc ksrc = head_src(a.kc, static_cast<const __bf16*>(a.kcur) + cel, a, h, D, 2, 2);
    const HeadSrc vsrc = head_src(a.vc, static_cast<const __bf16*>(a.vcur) + cel, a, h, D, 2, 2);
    const float c = a.scale_log2;  // base-2 softmax scale

    FetchRun fr = SEQ ? fetch_run_in(a, ur.rb, 0, shift) : fetch_run_at<DEVT>(a, 0);
    // real keys of a tile of this unit
    auto valid = [&](int tile) {
      return SEQ ? tile_valid_of(ur.ct, nkc, a.n, tile, C::BN) : tile_valid(a, tile, C::BN);
    };
    bf16_fetch_tile<D, SEQ, DEVT>(a, ksrc, vsrc, t0, fr, fl, smem, wave, ur);
    if (nt > 1) bf16_fetch_tile<D, SEQ, DEVT>(a, ksrc, vsrc, t0 + 1, fr, fl, smem + C::STAGE, wave, ur);

    // Q^T fragments (B operand): lane holds query q0+l32, dims 16kk+8hi .. +7;
    // rows past the chunk read as zeros (out-of-range buffer offsets).
    // Each wave group loads its Q in its own branch below (group 1 needs it a
    // phase later and waits for it then), so that the compiler, which sees
    // only these loads, places its one wait for them at a point of the
    // group's own code where no tile request it cannot see is in flight.
    const __bf16* qc = static_cast<const __bf16*>(a.q) + cel;
    const HeadSrc qsrc = head_src(qc, qc, a, h, D, 2, 2);
    auto load_q = [&](bf16x8_t (&qf)[D / 16]) {
      const int row = q0 + l32;
      const int qoff = row < a.n ? (row * a.H * D + 8 * hi) * 2 : kOob;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const uint4 x = buf16(qsrc.cur, qsrc.cur_bytes, qoff + (row < a.n ? 32 * kk : 0));
        qf[kk] = __builtin_bit_cast(bf16x8_t, x);
      }
    };

    PPState<D> st;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.o[db] = f32x16_t{};
    st.s[0] = f32x16_t{};
    st.s[1] = f32x16_t{};
#pragma unroll
    for (int e = 0; e < 4; ++e) st.pf[e] = bf16x8_t{};
    st.m_run = -INFINITY;
    st.l_run = 0.f;

    // Even phases 2r start by requesting tile r+2; odd phases 2q-1 end by
    // waiting for this wave's requests of tile q (read from phase 2q on).
    auto begin_phase = [&](int k) {
      const int r = k >> 1;
      if ((k & 1) == 0 && r + 2 < nt)
        bf16_fetch_tile<D, SEQ, DEVT>(a, ksrc, vsrc, t0 + r + 2, fr, fl, smem + ((r + 2) & 3) * C::STAGE,
                           wave, ur);
    };
    auto end_phase = [&](int k) {
      const int q = (k + 1) >> 1;
      if ((k & 1) == 1 && q < nt) {
        if (q + 1 < nt)
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::LOADS) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      wg_barrier();
    };
    auto stage = [&](int r) -> const unsigned char* { return smem + (r & 3) * C::STAGE; };

    if (grp == 0) {
      // Q and this wave's shares of the first two tiles, with a wait the
      // compiler sees: it then knows Q is loaded and inserts no vector-memory
      // waits in the loop, where the only loads in flight are the tile
      // requests this kernel waits for itself.
      bf16x8_t qf[D / 16];
      load_q(qf);
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      wg_barrier();
      // k = 2r: PV(r-1) + QK(r); k = 2r+1: softmax(r)
      begin_phase(0);
      if (wave_rows) {
        __builtin_amdgcn_s_setprio(1);
        pp_gemm<D, false, true>(st, nullptr, stage(0), koff, voff, qf);
        __builtin_amdgcn_s_setprio(0);
      }
      end_phase(0);
      begin_phase(1);
      if (wave_rows) pp_softmax<D>(st, valid(t0), hi, c);
      end_phase(1);
      for (int r = 1; r < nt; ++r) {
        begin_phase(2 * r);
        if (wave_rows) {
          __builtin_amdgcn_s_setprio(1);
          pp_gemm<D, true, true>(st, stage(r - 1), stage(r), koff, voff, qf);
          __builtin_amdgcn_s_setprio(0);
        }
        end_phase(2 * r);
        begin_phase(2 * r + 1);
        if (wave_rows) pp_softmax<D>(st, valid(t0 + r), hi, c);
        end_phase(2 * r + 1);
      }
      begin_phase(2 * nt);
      if (wave_rows) {
        __builtin_amdgcn_s_setprio(1);
        pp_gemm<D, true, false>(st, stage(nt - 1), nullptr, koff, voff, qf);
        __builtin_amdgcn_s_setprio(0);
      }
      end_phase(2 * nt);
      begin_phase(2 * nt + 1);
      end_phase(2 * nt + 1);
    } else {
      // Q after this wave's tile requests: the tiles' shares are waited for
      // before the first barrier (everything but the D/16 Q loads, which
      // complete in order after them), Q itself during phase 0, where this
      // group has nothing to compute, with a wait the compiler sees, before
      // the tile-2 requests are issued.
      bf16x8_t qf[D / 16];
      load_q(qf);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(D / 16) : "memory");
      wg_barrier();
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      // one phase later: k = 2r+1: PV(r-1) + QK(r); k = 2r+2: softmax(r)
      begin_phase(0);
      end_phase(0);
      begin_phase(1);
      if (wave_rows) {
        __builtin_amdgcn_s_setprio(1);
        pp_gemm<D, false, true>(st, nullptr, stage(0), koff, voff, qf);
        __builtin_amdgcn_s_setprio(0);
      }
      end_phase(1);
      for (int r = 1; r < nt; ++r) {
        begin_phase(2 * r);
        if (wave_rows) pp_softmax<D>(st, valid(t0 + r - 1), hi, c);
        end_phase(2 * r);
        begin_phase(2 * r + 1);
        if (wave_rows) {
          __builtin_amdgcn_s_setprio(1);
          pp_gemm<D, true, true>(st, stage(r - 1), stage(r), koff, voff, qf);
          __builtin_amdgcn_s_setprio(0);
        }
        end_phase(2 * r + 1);
      }
      begin_phase(2 * nt);
      if (wave_rows) pp_softmax<D>(st, valid(t0 + nt - 1), hi, c);
      end_phase(2 * nt);
      begin_phase(2 * nt + 1);
      if (wave_rows) {
        __builtin_amdgcn_s_setprio(1);
        pp_gemm<D, true, false>(st, stage(nt - 1), nullptr, koff, voff, qf);
        __builtin_amdgcn_s_setprio(0);
      }
      end_phase(2 * nt + 1);
    }

    // epilogue: normalise, LSE (natural log), write final output or a partial
    if (wave_rows) {
      const float l_tot = xhalf_sum(st.l_run);
      const float inv = 1.0f / l_tot;
      const float lse_val = (st.m_run + log2f(l_tot)) * kLn2;
      const int row = q0 + l32;
      const bool whole = (t0 == 0) && (t1 == T);
      if (whole) {
        // the wave's 32 rows through its own 32 rows of LDS stages 2-3 (free
        // here: the next unit requests tile 2 only after its first barrier),
        // so that every store writes whole rows (RPW rows of D bf16)
        constexpr int CPR = D / 8, RPW = 64 / CPR;
        // lane-derived offsets computed here, not kept through the tile loop
        int le = lane;
        asm volatile("" : "+v"(le));
        const int r32 = le & 31, h2 = le >> 5;
        unsigned char* ws = smem + 2 * C::STAGE + (wave & 7) * 32 * C::ROWB;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4_t v4 = {st.o[db][4 * g], st.o[db][4 * g + 1], st.o[db][4 * g + 2],
                          st.o[db][4 * g + 3]};
            v4 *= inv;
            *reinterpret_cast<bf16x4_t*>(ws + r32 * C::ROWB + (((4 * db + g) ^ (r32 % CPR)) << 4) +
                                         8 * h2) = __builtin_convertvector(v4, bf16x4_t);
          }
        const int rq = le / CPR, cq = le % CPR;
#pragma unroll
        for (int i = 0; i < 32 / RPW; ++i) {
          const int rr = i * RPW + rq;
          const uint4 x = *reinterpret_cast<const uint4*>(ws + rr * C::ROWB + ((cq ^ (rr % CPR)) << 4));
          if (q0 + rr < a.n)
            *reinterpret_cast<uint4*>(static_cast<__bf16*>(a.o) + cel +
                                      ((int64_t)(q0 + rr) * a.H + h) * D + 8 * cq) = x;
        }
        if (hi == 0 && a.lse && row < a.n)
          a.lse[(SEQ ? ci * a.chunk_lse : 0) + (int64_t)h * a.n + row] = lse_val;
      } else if (row < a.n) {
        const int64_t slot = SEQ ? part_slot_of(a, w, u, I) : part_slot(w, u, I, a.T, a.P, a.spw);
        const int64_t prow = slot * C::BM + (wave & 7) * 32 + l32;
        // fp16 partial outputs with a power-of-two scale per row: the row's
        // largest |O| (over the lane pair that holds the row) is brought into
        // [0.5, 1), so a value is rounded to within 2^-12 of that maximum
        // (bf16 would give 2^-9) in the same two bytes; the exponent goes to
        // part_exp and the merge multiplies it back exactly. A row with a
        // NaN or an infinity keeps exponent 0 and carries them through.
        // The wave's 32 rows are stored as the lanes hold them (chunk
        // 2 db + hf of lane l at 16 bytes x (64 (2 db + hf) + l) from the
        // wave's first row), so that each store writes 1 KB of consecutive
        // bytes; merge_lanes_kernel reads that layout.
        float mx = 0.f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(st.o[db][e]));
        mx = xhalf_max(mx) * inv;
        int ex = 0;
        if (mx > 0.f && mx <= 3.402823466e38f) (void)frexpf(mx, &ex);
        const float sc = __builtin_amdgcn_ldexpf(inv, -ex);
        _Float16* pp = reinterpret_cast<_Float16*>(a.part_o) + (prow - l32) * D + lane * 8;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            f32x8_t v8;
#pragma unroll
            for (int j = 0; j < 8; ++j) v8[j] = st.o[db][8 * hf + j] * sc;
            *reinterpret_cast<f16x8_t*>(pp + (2 * db + hf) * 512) =
                __builtin_convertvector(v8, f16x8_t);
          }
        if (hi == 0) {
          a.part_lse[prow] = lse_val;
          a.part_exp[prow] = ex;
        }
      }
    }
    it += t1 - t0;
  }
}

// ---------------------------------------------------------------------------
// fp8 e4m3 cache on the fp8 matrix cores (v_mfma_f32_32x32x64_f8f6f4).
//
// Same work decomposition, ping-pong schedule and softmax as the bf16 kernel;
// what changes is the data in LDS and the products:
//   - K and V tiles stay e4m3 in LDS (rows of d bytes, 16-byte chunks
//     XOR-swizzled per row), loaded straight from the cache (or from the
//     e4m3 copy of the current chunk) by the direct-to-LDS loads;
//   - Q is scaled once per unit by one factor per query row (448 / amax) and
//     written as two e4m3 terms, hi = e4m3(x) and lo = e4m3(x - hi) (about
//     eight significant bits together); the row's scale, the head's K scale
//     and the softmax scale make one per-lane constant, because a lane owns
//     one query row of S^T;
//   - S^T = K Q^T: per 32-key block and 64-dim step one 32x32x64 MFMA per
//     Q term, both into the same accumulator. In
//     that instruction byte j of A in lane m + 32h meets byte j of B in lane
//     n + 32h, so any consistent assignment of dims to (h, j) works: here
//     dims 64 ks + 32 h + j, i.e. 32 contiguous bytes of a row per lane;
//   - P is produced scaled by 2^4 (the exponent's +4 costs nothing) under a
//     running maximum that lags the true one by at most 4, so 0 <= P <= 2^8,
//     and written as two e4m3 terms like Q (one e4m3 term alone moves O by
//     several 1e-2 on data with 8-sigma outliers);
//   - O^T += V^T P^T: the MFMA's key index (h, j) with j = 16 kb + 4 a + b
//     is key 32 kb + 8 a + 4 h + b, the order in which the score layout
//     leaves a lane's 32 keys, so P^T is the lane's own scores in order;
//     V^T comes from transposing 8-bit LDS reads (ds_read_b64_tr_b8: within
//     16 lanes, lane i takes byte i % 8 of the 8 bytes addressed by lane
//     2r + (i >= 8), r = 0..7), four per 32-dim block.
// O is in units of the head's V scale; the output normalisation applies it.
template <int D>
struct F8Cfg {
  static constexpr int BM = 256, BN = 64, NSTAGE = 4;
  static constexpr int ROWB = D;                // bytes per key row
  static constexpr int CPR = D / 16;            // 16-byte chunks per row
  static constexpr int TILE_BYTES = BN * ROWB;  // K (or V) of one tile
  static constexpr int STAGE = 2 * TILE_BYTES;  // K then V
  static constexpr int RPL = 1024 / ROWB;       // rows per wave-wide 16-byte load
  static constexpr int LOADS = 2;               // requests per wave per tile (K, V)
  static constexpr int KS = D / 64;             // 64-dim steps of a score block
  static_assert(BN == 8 * RPL, "each of the 8 waves requests RPL rows of K and of V");
};

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;

// Physical 16-byte chunk of logical chunk c in row r is c ^ swizzle(r). K:
// the 32 rows one read instruction gathers spread over 8 chunk positions. V:
// the 8 rows one transposing read gathers (keys base + {0..3, 8..11}) take
// 8 different chunk positions.
__device__ __forceinline__ int f8_kswz(int r) { return r & 7; }
__device__ __forceinline__ int f8_vswz(int r) { return (r & 3) | (((r >> 3) & 1) << 2); }

// Requests the e4m3 rows of K and V of key tile `tile` into one stage. Lane L
// of wave w covers tile row RPL w + L / CPR and stage chunk L % CPR, which
// holds the row's logical chunk (L % CPR) ^ swizzle(row).
// This head's K and V sources: cache matrices and the rows of the e4m3 copy
// of the chunk ([H][n][d], row stride d).
struct F8Src {
  const char *kc, *vc, *kcur, *vcur;
  int cache_bytes, cur_bytes;
};

template <int D>
__device__ __forceinline__ F8Src f8_src(const AttnArgs& a, int h) {
  F8Src f;
  f.kc = uniform_ptr(static_cast<const char*>(a.kc) + (int64_t)h * a.cache_head_elems);
  f.vc = uniform_ptr(static_cast<const char*>(a.vc) + (int64_t)h * a.cache_head_elems);
  f.kcur = uniform_ptr(static_cast<const char*>(a.kcur) + (int64_t)h * a.n * D);
  f.vcur = uniform_ptr(static_cast<const char*>(a.vcur) + (int64_t)h * a.n * D);
  f.cache_bytes = (int)a.cache_span_elems;
  f.cur_bytes = a.n * D;
  return f;
}

template <int D, bool DEVT>
__device__ __forceinline__ void f8_fetch_tile(const AttnArgs& a, const F8Src& src, int tile,
                                              FetchRun& fr, unsigned char* stage, int wave,
                                              int lane) {
  using C = F8Cfg<D>;
  const int r = wave * C::RPL + lane / C::CPR;
  const int c = lane % C::CPR;
  const int kcol = (c ^ f8_kswz(r)) << 4, vcol = (c ^ f8_vswz(r)) << 4;
  unsigned char* kdst = stage + wave * 1024;
  unsigned char* vdst = kdst + C::TILE_BYTES;
  if (tile < a.cache_tiles) {
    const int j0 = tile * C::BN;
    while (j0 >= fr.vend && fr.ri + 1 < nruns_of<DEVT>(a)) fr = fetch_run_at<DEVT>(a, fr.ri + 1);
    int phys;
    if (j0 + C::BN <= fr.vend) {
      phys = fr.phys + j0 - fr.vstart + r;
    } else {
      const int j = j0 + r;
      phys = -1;
      for (int rr = fr.ri; rr < nruns_of<DEVT>(a); ++rr) {
        const Run R = run_of<DEVT>(a, rr);
        if (R.vstart >= j0 + C::BN) break;
        if (j >= R.vstart && j < R.vstart + R.len) phys = R.phys + j - R.vstart;
      }
    }
    lds_load16(src.kc, src.cache_bytes, phys >= 0 ? phys * D + kcol : kOob, kdst);
    lds_load16(src.vc, src.cache_bytes, phys >= 0 ? phys * D + vcol : kOob, vdst);
  } else {
    // rows past the chunk lie past the resource and read as zeros
    const int row = (tile - a.cache_tiles) * C::BN + r;
    lds_load16(src.kcur, src.cur_bytes, row * D + kcol, kdst);
    lds_load16(src.vcur, src.cur_bytes, row * D + vcol, vdst);
  }
}

// Four floats (within the e4m3 range) as two e4m3 words: [0] = hi =
// e4m3(x), [1] = lo = e4m3(x - hi), bytes in argument order.
__device__ __forceinline__ i32x2_t split_e4m3x4(float a, float b, float c, float d) {
  int x = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  x = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, x, true);
  const f32x2_t ab = __builtin_amdgcn_cvt_pk_f32_fp8(x, false);
  const f32x2_t cd = __builtin_amdgcn_cvt_pk_f32_fp8(x, true);
  int y = __builtin_amdgcn_cvt_pk_fp8_f32(a - ab[0], b - ab[1], 0, false);
  y = __builtin_amdgcn_cvt_pk_fp8_f32(c - cd[0], d - cd[1], y, true);
  return i32x2_t{x, y};
}

template <int D>
struct F8State {
  f32x16_t o[D / 32];  // O^T accumulator (layout of the bf16 kernel)
  f32x16_t s[2];       // S^T of the tile, keys 0-31 and 32-63
  i32x8_t pf[2];       // P^T of the tile (x 2^8) as e4m3 hi and lo terms, between softmax and PV
  float m_run, l_run;  // running maximum (base 2) and this lane's partial sum (x 2^8)
};

// One MFMA phase of the fp8 kernel: PV of the tile in stage SV (per 32-dim
// block, one MFMA per P term) and/or QK of the tile in stage SK (per key block
// and 64-dim step, one MFMA per Q term). Step i issues PV hi, QK hi, PV lo,
// QK lo with the operands loaded one step ahead.
template <int D, bool PV, bool QK>
__device__ __forceinline__ void f8_gemm(F8State<D>& st, const unsigned char* SV,
                                        const unsigned char* SK, const int (&koff)[2 * (D / 64)],
                                        const int (&voff)[D / 32],
                                        const i32x8_t (&qf)[2][D / 64]) {
  using C = F8Cfg<D>;
  constexpr int NPV = PV ? D / 32 : 0;
  constexpr int NQK = QK ? 2 * C::KS : 0;
  constexpr int NSTEP = NPV > NQK ? NPV : NQK;
  i32x8_t vf[NSTEP + 1], kf[NSTEP + 1];
  auto load_v = [&](int i) {
    if (i < NPV) {
      const unsigned char* vp = SV + voff[i];
      i32x2_t t4[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        t4[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vp + 2048 * t));
      vf[i] = i32x8_t{t4[0][0], t4[0][1], t4[1][0], t4[1][1],
                      t4[2][0], t4[2][1], t4[3][0], t4[3][1]};
    }
  };
  auto load_k = [&](int i) {
    if (i < NQK) {
      // step i: key block i % 2, dim step i / 2
      const int kb = i & 1, ks = i >> 1;
      const unsigned char* kp = SK + kb * 32 * C::ROWB;
      const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(kp + koff[2 * ks]);
      const i32x4_t h4 = *reinterpret_cast<const i32x4_t*>(kp + koff[2 * ks + 1]);
      kf[i] = i32x8_t{lo[0], lo[1], lo[2], lo[3], h4[0], h4[1], h4[2], h4[3]};
    }
  };
  f32x16_t acc0 = f32x16_t{}, acc1 = f32x16_t{};
  load_v(0);
  load_k(0);
  __builtin_amdgcn_sched_barrier(0);
  auto mf = [](const i32x8_t& x, const i32x8_t& y, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 0, 0, 0);
  };
#pragma unroll
  for (int i = 0; i < NSTEP; ++i) {
    load_v(i + 1);
    load_k(i + 1);
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      if (i < NPV) st.o[i] = mf(vf[i], st.pf[part], st.o[i]);
      if (i < NQK) {
        if (i & 1)
          acc1 = mf(kf[i], qf[part][i >> 1], acc1);
        else
          acc0 = mf(kf[i], qf[part][i >> 1], acc0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (QK) {
    st.s[0] = acc0;
    st.s[1] = acc1;
  }
}

typedef int i32x16_t __attribute__((ext_vector_type(16)));

// INT8K_FP8V_BLOCK: the same phase with Q K^T on the int8 matrix cores
// (v_mfma_i32_32x32x32_i8, 16 bytes of A and B per lane). The 32 K bytes a
// lane holds per key block and 64-dim step (dims 64 ks + 32 h .. + 31, as for
// e4m3) feed two 32-deep MFMAs against the same dims of the Q terms. Pass 1
// takes Q's hi term into int32 accumulators, which are then shifted by 8 (lo
// counts 2^-8 of hi's unit); pass 2 adds the lo term. A score is thus
// sum_d k (256 hi + lo), exact in int32 (at most 127 * 32639 * D < 2^31 for
// D = 128), and is converted to float once. P V is the fp8 kernel's.
template <int D, bool PV, bool QK>
__device__ __forceinline__ void i8_gemm(F8State<D>& st, const unsigned char* SV,
                                        const unsigned char* SK, const int (&koff)[2 * (D / 64)],
                                        const int (&voff)[D / 32],
                                        const i32x8_t (&qf)[2][D / 64]) {
  using C = F8Cfg<D>;
  constexpr int NPV = PV ? D / 32 : 0;
  constexpr int NQK = QK ? 2 * C::KS : 0;
  constexpr int NSTEP = NPV > NQK ? NPV : NQK;
  i32x8_t vf[NSTEP + 1], kf[NSTEP + 1];
  auto load_v = [&](int i) {
    if (i < NPV) {
      const unsigned char* vp = SV + voff[i];
      i32x2_t t4[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        t4[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vp + 2048 * t));
      vf[i] = i32x8_t{t4[0][0], t4[0][1], t4[1][0], t4[1][1],
                      t4[2][0], t4[2][1], t4[3][0], t4[3][1]};
    }
  };
  auto load_k = [&](int i) {
    if (i < NQK) {
      const int kb = i & 1, ks = i >> 1;
      const unsigned char* kp = SK + kb * 32 * C::ROWB;
      const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(kp + koff[2 * ks]);
      const i32x4_t h4 = *reinterpret_cast<const i32x4_t*>(kp + koff[2 * ks + 1]);
      kf[i] = i32x8_t{lo[0], lo[1], lo[2], lo[3], h4[0], h4[1], h4[2], h4[3]};
    }
  };
  auto mf = [](const i32x8_t& x, const i32x8_t& y, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 0, 0, 0);
  };
  // the two 16-byte halves of a lane's 32 bytes: dims +0..15 and +16..31
  auto mi = [](const i32x8_t& x, const i32x8_t& y, int half, const i32x16_t& c) {
    const i32x4_t xa = half ? i32x4_t{x[4], x[5], x[6], x[7]} : i32x4_t{x[0], x[1], x[2], x[3]};
    const i32x4_t ya = half ? i32x4_t{y[4], y[5], y[6], y[7]} : i32x4_t{y[0], y[1], y[2], y[3]};
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(xa, ya, c, 0, 0, 0);
  };
  i32x16_t acc0 = i32x16_t{}, acc1 = i32x16_t{};
  load_v(0);
  load_k(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NSTEP; ++i) {
    load_v(i + 1);
    load_k(i + 1);
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      if (i < NPV) st.o[i] = mf(vf[i], st.pf[part], st.o[i]);
      if (i < NQK) {
        if (i & 1)
          acc1 = mi(kf[i], qf[0][i >> 1], part, acc1);
        else
          acc0 = mi(kf[i], qf[0][i >> 1], part, acc0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (QK) {
    // pass 2 reads the K fragments from LDS again (the stage stays valid until
    // the phase's barrier) rather than holding all of them in registers
    i32x8_t kg[NQK + 1];
    auto reload_k = [&](int i) {
      if (i < NQK) {
        const int kb = i & 1, ks = i >> 1;
        const unsigned char* kp = SK + kb * 32 * C::ROWB;
        const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(kp + koff[2 * ks]);
        const i32x4_t h4 = *reinterpret_cast<const i32x4_t*>(kp + koff[2 * ks + 1]);
        kg[i] = i32x8_t{lo[0], lo[1], lo[2], lo[3], h4[0], h4[1], h4[2], h4[3]};
      }
    };
    reload_k(0);
    acc0 <<= 8;
    acc1 <<= 8;
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      reload_k(i + 1);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if (i & 1)
          acc1 = mi(kg[i], qf[1][i >> 1], half, acc1);
        else
          acc0 = mi(kg[i], qf[1][i >> 1], half, acc0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    st.s[0] = __builtin_convertvector(acc0, f32x16_t);
    st.s[1] = __builtin_convertvector(acc1, f32x16_t);
  }
}

template <int D, bool I8K, bool PV, bool QK>
__device__ __forceinline__ void x8_gemm(F8State<D>& st, const unsigned char* SV,
                                        const unsigned char* SK, const int (&koff)[2 * (D / 64)],
                                        const int (&voff)[D / 32],
                                        const i32x8_t (&qf)[2][D / 64]) {
  if constexpr (I8K)
    i8_gemm<D, PV, QK>(st, SV, SK, koff, voff, qf);
  else
    f8_gemm<D, PV, QK>(st, SV, SK, koff, voff, qf);
}

// Online softmax of the fp8 kernel's tile, c per lane (the query row's scale
// included). The running maximum moves only when a tile exceeds it by more
// than 4; P is scaled by 2^4, so P <= 2^8 stays within e4m3 and values down
// to 2^-13 of the row's maximum keep a normal e4m3 representation.
template <int D>
// off_add and sum_fac serve caches with one scale per block (per tile): P
// comes out multiplied by 2^off_add = s_V(tile) / s_ref <= 1, and the row
// sum gets the tile's weights divided back by that ratio (sum_fac).
__device__ __forceinline__ void f8_softmax(F8State<D>& st, int lim, int hi, float c,
                                           float off_add = 0.f, float sum_fac = 1.f) {
  if (lim < 64) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kr = 8 * (e >> 2) + 4 * hi + (e & 3);
      if (kr >= lim) st.s[0][e] = -INFINITY;
      if (32 + kr >= lim) st.s[1][e] = -INFINITY;
    }
  }
  const f32x16_t v0 = st.s[0], v1 = st.s[1];
  float m[11];
#pragma unroll
  for (int e = 0; e < 5; ++e) m[e] = max3n(v0[3 * e], v0[3 * e + 1], v0[3 * e + 2]);
#pragma unroll
  for (int e = 0; e < 5; ++e) m[5 + e] = max3n(v1[3 * e], v1[3 * e + 1], v1[3 * e + 2]);
  m[10] = __builtin_elementwise_maximum(v0[15], v1[15]);
  const float n0 = max3n(m[0], m[1], m[2]), n1 = max3n(m[3], m[4], m[5]);
  const float n2 = max3n(m[6], m[7], m[8]), n3 = __builtin_elementwise_maximum(m[9], m[10]);
  // c > 0, so the maximum of the scaled scores is c times the maximum score
  const float mxs = xhalf_maxn(max3n(n0, n1, __builtin_elementwise_maximum(n2, n3)) * c);
  if (__any(!(mxs <= st.m_run + 4.0f))) {
    const float m_new = fmaxf(st.m_run, mxs);
    const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.o[db] *= alpha;
    st.l_run *= alpha;
    st.m_run = m_new;
  }
  // P x 2^4 = 2^(s c - m + 4): at most 2^8
  const float off = (st.m_run == -INFINITY ? 4.f : 4.f - st.m_run) + off_add;
  f32x16_t p0, p1;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    p0[e] = __builtin_amdgcn_exp2f(fmaf(v0[e], c, off));
    p1[e] = __builtin_amdgcn_exp2f(fmaf(v1[e], c, off));
  }
  float t8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) t8[e] = (p0[e] + p0[e + 8]) + (p1[e] + p1[e + 8]);
  st.l_run += (((t8[0] + t8[4]) + (t8[1] + t8[5])) + ((t8[2] + t8[6]) + (t8[3] + t8[7]))) *
              sum_fac;
  // byte j = 16 kb + e of P^T holds key block kb's score e
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const i32x2_t s0 = split_e4m3x4(p0[4 * w], p0[4 * w + 1], p0[4 * w + 2], p0[4 * w + 3]);
    const i32x2_t s1 = split_e4m3x4(p1[4 * w], p1[4 * w + 1], p1[4 * w + 2], p1[4 * w + 3]);
    st.pf[0][w] = s0[0];
    st.pf[1][w] = s0[1];
    st.pf[0][4 + w] = s1[0];
    st.pf[1][4 + w] = s1[1];
  }
}

// BLK: an FP8_E4M3_BLOCK cache. Every visible block is its own run padded to
// whole key tiles, so each tile has one block's K and V scales: the K scale
// multiplies the tile's softmax constant, and the V scale relative to the
// unit's largest (s_ref) enters P as an exponent offset, with the row sum
// corrected per tile and s_ref applied at normalisation.
template <int D, bool BLK, bool DEVT, bool I8K = false>
__global__ __launch_bounds__(512) void attn_fp8_kernel(const AttnArgs a) {
  static_assert(!I8K || BLK, "int8 K comes with per-block scales");
  using C = F8Cfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::NSTAGE * C::STAGE];
  // BLK: the unit's K scale per block, and per block the exponent offset
  // log2(s_V / s_ref) and the row-sum factor s_ref / s_V
  __shared__ float sc_k[kMaxBlocks], sc_off[kMaxBlocks], sc_fac[kMaxBlocks];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int w = logical_wg(a);
  const int64_t I = (int64_t)a.units * a.T;
  int64_t it = range_begin(w, I, a.P);
  const int64_t it_end = range_begin(w + 1, I, a.P);

  // K operand: key row l32 (+32 per key block), 32 bytes at dims 64 ks + 32 hi
  int koff[2 * C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
    for (int x = 0; x < 2; ++x)
      koff[2 * ks + x] = l32 * C::ROWB + (((4 * ks + 2 * hi + x) ^ f8_kswz(l32)) << 4);
  // V^T operand of dim block db: lane 16 g + 2 r + s supplies the address of
  // key 8 (r / 4) + 4 hi + r % 4 (+ 16 t for read t), dims 32 db + 16 (g % 2)
  // + 8 s .. + 7
  int voff[D / 32];
  {
    const int ii = lane & 15, g2 = (lane >> 4) & 1, r = ii >> 1, sx = ii & 1;
    const int key = 8 * (r >> 2) + 4 * hi + (r & 3);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      voff[db] = C::TILE_BYTES + key * C::ROWB + (((2 * db + g2) ^ f8_vswz(key)) << 4) + 8 * sx;
  }

  if constexpr (DEVT) {
    if (tid == 0) build_dev_runs<BLK>(a);
    __syncthreads();
  }
  while (it < it_end) {
    const int u = (int)(it / a.T);
    const int t0 = (int)(it - (int64_t)u * a.T);
    const int t1 = (int)((it_end - it) < (int64_t)(a.T - t0) ? t0 + (it_end - it) : a.T);
    const int nt = t1 - t0;
    const int h = __builtin_amdgcn_readfirstlane(u / a.QT);
    const int qt = u - h * a.QT;
    const int q0 = qt * C::BM + (wave & 7) * 32;
    const bool wave_rows = q0 < a.n;

    FetchRun fr = fetch_run_at<DEVT>(a, 0);
    const F8Src src = f8_src<D>(a, h);
    f8_fetch_tile<D, DEVT>(a, src, t0, fr, smem, wave, lane);
    if (nt > 1) f8_fetch_tile<D, DEVT>(a, src, t0 + 1, fr, smem + C::STAGE, wave, lane);

    // Q: lane holds row q0 + l32, dims 64 ks + 32 hi .. + 31 (bf16); rows
    // past the chunk read as zeros. Quantised with the row's scale amax/448.
    const HeadSrc qsrc = head_src(a.q, a.q, a, h, D, 2, 2);
    i32x8_t qf[2][C::KS];
    float c;
    {
      const int row = q0 + l32;
      uint4 raw[4 * C::KS];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int x = 0; x < 4; ++x)
          raw[4 * ks + x] = buf16(qsrc.cur, qsrc.cur_bytes,
                                  row < a.n ? (row * a.H * D + 64 * ks + 32 * hi + 8 * x) * 2
                                            : kOob);
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      float amax = 0.f;
#pragma unroll
      for (int x = 0; x < 4 * C::KS; ++x) {
        const bf16x8_t v = __builtin_bit_cast(bf16x8_t, raw[x]);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)v[e]));
      }
      amax = xhalf_max(amax);
      if constexpr (I8K) {
        // two int8 terms per element: y = x 127 / amax, hi = rne(y), lo =
        // rne(256 (y - hi)) (y - hi is exact), so x = (amax / 127)(hi + lo / 256)
        // to within 2^-9 of the row's code unit
        const float qs = amax > 0.f ? amax / 127.0f : 1.0f;
        const float qinv = amax > 0.f ? 127.0f / amax : 1.0f;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const bf16x8_t v = __builtin_bit_cast(bf16x8_t, raw[4 * ks + x]);
            unsigned wh[2] = {0u, 0u}, wl[2] = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float y = fminf(fmaxf((float)v[e] * qinv, -127.f), 127.f);
              const float hq = __builtin_rintf(y);
              const float lq = fminf(fmaxf(__builtin_rintf((y - hq) * 256.0f), -127.f), 127.f);
              wh[e >> 2] |= ((unsigned)(int)hq & 0xffu) << (8 * (e & 3));
              wl[e >> 2] |= ((unsigned)(int)lq & 0xffu) << (8 * (e & 3));
            }
            qf[0][ks][2 * x] = (int)wh[0];
            qf[0][ks][2 * x + 1] = (int)wh[1];
            qf[1][ks][2 * x] = (int)wl[0];
            qf[1][ks][2 * x + 1] = (int)wl[1];
          }
        // an int32 score is 256 / qs times the products in the K codes' unit
        c = a.scale_log2 * qs * (1.0f / 256.0f);
      } else {
        const float qs = amax > 0.f ? amax * (1.0f / 448.0f) : 1.0f;
        const float qinv = amax > 0.f ? 448.0f / amax : 1.0f;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const bf16x8_t v = __builtin_bit_cast(bf16x8_t, raw[4 * ks + x]);
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = fminf(fmaxf((float)v[e] * qinv, -448.f), 448.f);
            const i32x2_t lo4 = split_e4m3x4(f[0], f[1], f[2], f[3]);
            const i32x2_t hi4 = split_e4m3x4(f[4], f[5], f[6], f[7]);
            qf[0][ks][2 * x] = lo4[0];
            qf[1][ks][2 * x] = lo4[1];
            qf[0][ks][2 * x + 1] = hi4[0];
            qf[1][ks][2 * x + 1] = hi4[1];
          }
        // base-2 scale of the raw products: softmax scale, K scale, Q row scale
        // (BLK: the K scale comes per tile)
        c = BLK ? a.scale_log2 * qs : a.scale_log2 * a.k_scale[h] * qs;
      }
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    float sv_ref = 1.f;
    if constexpr (BLK) {
      // the visible blocks' scales of this head, then the current chunk's
      float svj = 0.f;
      if (tid <= a.nvis_cache) {
        const bool cur = tid == a.nvis_cache;
        const int64_t e = cur ? h : (int64_t)(DEVT ? dev_vis[tid] : a.vis_blk[tid]) * a.H + h;
        sc_k[tid] = cur ? a.cur_sc[e] : a.ksc[e];
        svj = cur ? a.cur_sc[a.H + e] : a.vsc[e];
        sc_fac[tid] = svj;
      }
      __syncthreads();
      sv_ref = sc_fac[0];
      for (int j = 1; j <= a.nvis_cache; ++j) sv_ref = fmaxf(sv_ref, sc_fac[j]);
      __syncthreads();
      if (tid <= a.nvis_cache) {
        sc_off[tid] = __log2f(svj / sv_ref);
        sc_fac[tid] = sv_ref / svj;
      }
      __syncthreads();
    }

    F8State<D> st;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.o[db] = f32x16_t{};
    st.s[0] = f32x16_t{};
    st.s[1] = f32x16_t{};
    st.pf[0] = i32x8_t{};
    st.pf[1] = i32x8_t{};
    st.m_run = -INFINITY;
    st.l_run = 0.f;

    // softmax of tile tt (BLK: with its block's scales). Each wave visits the
    // unit's tiles in increasing order, so the block of a cache tile is
    // tracked from the unit's first tile on instead of divided out per tile.
    int blk_j = BLK ? t0 / a.tpb : 0, blk_end = BLK ? (blk_j + 1) * a.tpb : 0;
    auto softmax_tile = [&](int tt) {
      if constexpr (BLK) {
        const bool cache_tile = tt < a.cache_tiles;
        while (tt >= blk_end) {
          ++blk_j;
          blk_end += a.tpb;
        }
        const int j = cache_tile ? blk_j : a.nvis_cache;
        const int lim = cache_tile ? min(C::BN, a.n - C::BN * (tt - (blk_end - a.tpb)))
                                   : tile_valid(a, tt, C::BN);
        f8_softmax<D>(st, lim, hi, c * sc_k[j], sc_off[j], sc_fac[j]);
      } else {
        f8_softmax<D>(st, tile_valid(a, tt, C::BN), hi, c);
      }
    };

    // Even phases 2r start by requesting tile r+2; odd phases 2q-1 end by
    // waiting for this wave's requests of tile q (read from phase 2q on).
    auto begin_phase = [&](int k) {
      if ((k & 1) == 0 && (k >> 1) + 2 < nt)
        f8_fetch_tile<D, DEVT>(a, src, t0 + (k >> 1) + 2, fr, smem + (((k >> 1) + 2) & 3) * C::STAGE,
                         wave, lane);
    };
    auto end_phase = [&](int k) {
      const int q = (k + 1) >> 1;
      if ((k & 1) == 1 && q < nt) {
        if (q + 1 < nt)
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::LOADS) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      wg_barrier();
    };
    auto stage = [&](int r) -> const unsigned char* { return smem + (r & 3) * C::STAGE; };

    wg_barrier();

    if (grp == 0) {
      begin_phase(0);
      if (wave_rows) {
        __builtin_amdgcn_s_setprio(1);
        x8_gemm<D, I8K, false, true>(st, nullptr, stage(0), koff, voff, qf);
        __builtin_amdgcn_s_setprio(0);
      }
      end_phase(0);
      begin_phase(1);
      if (wave_rows) softmax_tile(t0);
      end_phase(1);
      for (int r = 1; r < nt; ++r) {
        begin_phase(2 * r);
        if (wave_rows) {
          __builtin_amdgcn_s_setprio(1);
          x8_gemm<D, I8K, true, true>(st, stage(r - 1), stage(r), koff, voff, qf);
          __builtin_amdgcn_s_setprio(0);
        }
        end_phase(2 * r);
        begin_phase(2 * r + 1);
        if (wave_rows) softmax_tile(t0 + r);
        end_phase(2 * r + 1);
      }
      begin_phase(2 * nt);
      if (wave_rows) {
        __builtin_amdgcn_s_setprio(1);
        x8_gemm<D, I8K, true, false>(st, stage(nt - 1), nullptr, koff, voff, qf);
        __builtin_amdgcn_s_setprio(0);
      }
      end_phase(2 * nt);
      begin_phase(2 * nt + 1);
      end_phase(2 * nt + 1);
    } else {
      begin_phase(0);
      end_phase(0);
      begin_phase(1);
      if (wave_rows) {
        __builtin_amdgcn_s_setprio(1);
        x8_gemm<D, I8K, false, true>(st, nullptr, stage(0), koff, voff, qf);
        __builtin_amdgcn_s_setprio(0);
      }
      end_phase(1);
      for (int r = 1; r < nt; ++r) {
        begin_phase(2 * r);
        if (wave_rows) softmax_tile(t0 + r - 1);
        end_phase(2 * r);
        begin_phase(2 * r + 1);
        if (wave_rows) {
          __builtin_amdgcn_s_setprio(1);
          x8_gemm<D, I8K, true, true>(st, stage(r - 1), stage(r), koff, voff, qf);
          __builtin_amdgcn_s_setprio(0);
        }
        end_phase(2 * r + 1);
      }
      begin_phase(2 * nt);
      if (wave_rows) softmax_tile(t0 + nt - 1);
      end_phase(2 * nt);
      begin_phase(2 * nt + 1);
      if (wave_rows) {
        __builtin_amdgcn_s_setprio(1);
        x8_gemm<D, I8K, true, false>(st, stage(nt - 1), nullptr, koff, voff, qf);
        __builtin_amdgcn_s_setprio(0);
      }
      end_phase(2 * nt + 1);
    }

    // epilogue: P carried 2^4 (in l and in O alike); O is in V-scale units
    if (wave_rows) {
      const float l_tot = xhalf_sum(st.l_run);
      const float inv = (BLK ? sv_ref : a.v_scale[h]) / l_tot;
      const float lse_val = (st.m_run - 4.0f + log2f(l_tot)) * kLn2;
      const int row = q0 + l32;
      const bool whole = (t0 == 0) && (t1 == a.T);
      if (row < a.n) {
        if (whole) {
          __bf16* op = static_cast<__bf16*>(a.o) + ((int64_t)row * a.H + h) * D;
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              f32x4_t v4 = {st.o[db][4 * g], st.o[db][4 * g + 1], st.o[db][4 * g + 2],
                            st.o[db][4 * g + 3]};
              v4 *= inv;
              *reinterpret_cast<bf16x4_t*>(op + 32 * db + 8 * g + 4 * hi) =
                  __builtin_convertvector(v4, bf16x4_t);
            }
          if (hi == 0 && a.lse) a.lse[(int64_t)h * a.n + row] = lse_val;
        } else {
          // fp16 partials scaled per row, stored as the lanes hold them: the
          // bf16 kernel's format, merged by merge_lanes_kernel
          const int64_t prow =
              part_slot(w, u, I, a.T, a.P, a.spw) * C::BM + (wave & 7) * 32 + l32;
          float mx = 0.f;
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(st.o[db][e]));
          mx = xhalf_max(mx) * inv;
          int ex = 0;
          if (mx > 0.f && mx <= 3.402823466e38f) (void)frexpf(mx, &ex);
          const float sc = __builtin_amdgcn_ldexpf(inv, -ex);
          _Float16* pp = reinterpret_cast<_Float16*>(a.part_o) + (prow - l32) * D + lane * 8;
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              f32x8_t v8;
#pragma unroll
              for (int j = 0; j < 8; ++j) v8[j] = st.o[db][8 * hf + j] * sc;
              *reinterpret_cast<f16x8_t*>(pp + (2 * db + hf) * 512) =
                  __builtin_convertvector(v8, f16x8_t);
            }
          if (hi == 0) {
            a.part_lse[prow] = lse_val;
            a.part_exp[prow] = ex;
          }
        }
      }
    }
    it += t1 - t0;
  }
}

// ---------------------------------------------------------------------------
// fp32 attention on the vector ALUs (the fp32 configuration is small; this
// kernel aims at exact agreement rather than throughput).
// Work group: 128 threads, BM = 64 rows, two threads per row each owning half
// of the head dimension; key tiles of 32 in LDS.
template <int D>
__global__ __launch_bounds__(128) void attn_f32_kernel(const AttnArgs a) {
  constexpr int BM = 64, BN = 32, NT = 128, HALF = D / 2;
  constexpr int CPR = D / 4;               // float4 per row
  constexpr int NCH = BN * CPR / NT;       // float4 loads per thread per tile (K and V each)
  __shared__ __attribute__((aligned(16))) float Ks[BN][D];
  __shared__ __attribute__((aligned(16))) float Vs[BN][D];

  const int tid = threadIdx.x;
  const int rloc = tid >> 1, half = tid & 1;
  const int w = logical_wg(a);
  const int64_t I = (int64_t)a.units * a.T;
  int64_t it = range_begin(w, I, a.P);
  const int64_t it_end = range_begin(w + 1, I, a.P);

  while (it < it_end) {
    const int u = (int)(it / a.T);
    const int t0 = (int)(it - (int64_t)u * a.T);
    const int t1 = (int)((it_end - it) < (int64_t)(a.T - t0) ? t0 + (it_end - it) : a.T);
    const int h = u / a.QT, qt = u - h * a.QT;
    const int row = qt * BM + rloc;

    float q[HALF], o[HALF];
    {
      const float* qp = static_cast<const float*>(a.q) + ((int64_t)min(row, a.n - 1) * a.H + h) * D +
                        half * HALF;
#pragma unroll
      for (int c = 0; c < HALF; c += 4) {
        f32x4_t v = *reinterpret_cast<const f32x4_t*>(qp + c);
        q[c] = v[0], q[c + 1] = v[1], q[c + 2] = v[2], q[c + 3] = v[3];
      }
#pragma unroll
      for (int c = 0; c < HALF; ++c) o[c] = 0.f;
    }
    float m_run = -INFINITY, l_run = 0.f;
    int ri = 0;
    const HeadSrc ksrc = head_src(a.kc, a.kcur, a, h, D, 4, 4);
    const HeadSrc vsrc = head_src(a.vc, a.vcur, a, h, D, 4, 4);

    for (int tile = t0; tile < t1; ++tile) {
      const int j0 = tile * BN;
      const int lim = tile_valid(a, tile, BN);
      int jr[NCH], cr[NCH];
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        jr[i] = (tid + NT * i) / CPR;  // row inside the tile
        cr[i] = (tid + NT * i) % CPR;
      }
      // every thread's chunks share one column: NT is a multiple of CPR
      uint4 kv[NCH], vv[NCH];
      if (tile < a.cache_tiles) {
        ri = advance_run(a, ri, j0);
        int jc[NCH];
#pragma unroll
        for (int i = 0; i < NCH; ++i) jc[i] = j0 + jr[i];
        load_cache_rows<NCH, BN>(a, ksrc, D, 4, j0, ri, jc, cr[0] * 16, kv);
        load_cache_rows<NCH, BN>(a, vsrc, D, 4, j0, ri, jc, cr[0] * 16, vv);
      } else {
        const int r0 = (tile - a.cache_tiles) * BN;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const int row = r0 + jr[i];
          const int off = row < a.n ? row * a.H * D * 4 + cr[i] * 16 : kOob;
          kv[i] = buf16(ksrc.cur, ksrc.cur_bytes, off);
          vv[i] = buf16(vsrc.cur, vsrc.cur_bytes, off);
        }
      }
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        *reinterpret_cast<uint4*>(&Ks[jr[i]][4 * cr[i]]) = kv[i];
        *reinterpret_cast<uint4*>(&Vs[jr[i]][4 * cr[i]]) = vv[i];
      }
      __syncthreads();

      float s[BN];
#pragma unroll
      for (int j = 0; j < BN; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < HALF; ++c) acc = fmaf(q[c], Ks[j][half * HALF + c], acc);
        acc += __shfl_xor(acc, 1);
        s[j] = (j < lim) ? acc * a.scale_log2 : -INFINITY;
      }
      float mx = s[0];
#pragma unroll
      for (int j = 1; j < BN; ++j) mx = fmaxf(mx, s[j]);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < HALF; ++c) o[c] *= alpha;
      m_run = m_new;
#pragma unroll
      for (int j = 0; j < BN; ++j) {
        const float p = exp2f(s[j] - m_run);
        l_run += p;
#pragma unroll
        for (int c = 0; c < HALF; ++c) o[c] = fmaf(p, Vs[j][half * HALF + c], o[c]);
      }
      __syncthreads();
    }

    if (row < a.n) {
      const float inv = 1.0f / l_run;
      const float lse_val = (m_run + log2f(l_run)) * kLn2;
      const bool whole = (t0 == 0) && (t1 == a.T);
      float* dst;
      if (whole) {
        dst = static_cast<float*>(a.o) + ((int64_t)row * a.H + h) * D + half * HALF;
        if (half == 0 && a.lse) a.lse[(int64_t)h * a.n + row] = lse_val;
      } else {
        const int64_t prow = part_slot(w, u, I, a.T, a.P, a.spw) * BM + rloc;
        dst = a.part_o + prow * D + half * HALF;
        if (half == 0) a.part_lse[prow] = lse_val;
      }
#pragma unroll
      for (int c = 0; c < HALF; c += 4) {
        f32x4_t v = {o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv};
        *reinterpret_cast<f32x4_t*>(dst + c) = v;
      }
    }
    it += t1 - t0;
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the segments of every split unit:
//   M = max_g LSE_g, w_g = exp(LSE_g - M) (0 for LSE_g = -inf),
//   O = sum_g w_g O_g / sum_g w_g, LSE = M + ln sum_g w_g.
// merge_kernel reads the fp32 path's partials, stored row by row: one work
// group covers 256 / (D/16) rows of one unit, each thread sixteen dims. The unit's first piece and piece count come from the range
// arithmetic once per work group (thread 0, through LDS).
// Pieces whose loads the merge issues all at once.
constexpr int kMergeBatch = 4;
constexpr int kMergeEpt = 16;  // dims per thread

// Eight fp32 partial-output values (fp32 path).
__device__ __forceinline__ void load_part8(const float* p, float (&x)[8]) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
  const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}
template <int D, typename OutT>
__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a) {
  constexpr int NG = kMergeEpt / 8, TPR = D / kMergeEpt, RPB = 256 / TPR;
  const int blocks_per_unit = (a.bm + RPB - 1) / RPB;
  const int u = blockIdx.x / blocks_per_unit;
  const int rb = blockIdx.x - u * blocks_per_unit;
  // pieces of unit u: the work groups w0 .. w0 + pieces - 1 whose ranges meet
  // it; piece j >= 1 has the slot of its own (its range starts inside unit u),
  // piece 0 part_slot's choice
  __shared__ int64_t s_w0, s_slot0;
  __shared__ int s_pieces;
  if (threadIdx.x == 0) {
    const int64_t I = (int64_t)a.units * a.T;
    const int64_t w0 = first_wg_of((int64_t)u * a.T, I, a.P);
    s_w0 = w0;
    s_pieces = (int)(first_wg_of((int64_t)(u + 1) * a.T - 1, I, a.P) - w0 + 1);
    s_slot0 = part_slot(w0, u, I, a.T, a.P, a.spw);
  }
  __syncthreads();
  const int pieces = s_pieces;
  if (pieces <= 1) return;  // written whole by the attention kernel
  const int rloc = rb * RPB + threadIdx.x / TPR;
  const int c8 = (threadIdx.x % TPR) * kMergeEpt;
  if (rloc >= a.bm) return;
  const int ci = u / a.upc, ul = u - ci * a.upc;  // chunk of a batched launch
  const int h = ul / a.QT, qt = ul - h * a.QT;
  const int row = qt * a.bm + rloc;
  if (row >= a.n) return;
  const int64_t w0 = s_w0;
  const int64_t prow0 = s_slot0 * a.bm + rloc;
  auto prow_of = [&](int j) -> int64_t {
    return j == 0 ? prow0 : ((w0 + j) * a.spw) * a.bm + rloc;
  };
  const float* part = a.part_o;
  float M = -INFINITY, wsum = 0.f;
  float acc[8 * NG];
#pragma unroll
  for (int i = 0; i < 8 * NG; ++i) acc[i] = 0.f;
  if (pieces <= kMergeBatch) {
    // every load of the row first, then the combination (one memory latency)
    float lj[kMergeBatch];
    float oj[kMergeBatch][8 * NG];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      if (j < pieces) {
        const int64_t prow = prow_of(j);
        lj[j] = a.part_lse[prow];
#pragma unroll
        for (int g = 0; g < NG; ++g)
          load_part8(part + prow * D + c8 + 8 * g, *reinterpret_cast<float(*)[8]>(&oj[j][8 * g]));
      }
    }
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
      if (j < pieces) M = fmaxf(M, lj[j]);
    if (M != -INFINITY) {
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) {
        if (j < pieces) {
          const float wj = (lj[j] == -INFINITY) ? 0.f : expf(lj[j] - M);
          wsum += wj;
#pragma unroll
          for (int i = 0; i < 8 * NG; ++i) acc[i] += wj * oj[j][i];
        }
      }
    }
  } else {
    for (int j = 0; j < pieces; ++j) M = fmaxf(M, a.part_lse[prow_of(j)]);
    if (M != -INFINITY) {
      for (int j = 0; j < pieces; ++j) {
        const int64_t prow = prow_of(j);
        const float lj = a.part_lse[prow];
        const float wj = (lj == -INFINITY) ? 0.f : expf(lj - M);
        wsum += wj;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          float oj[8];
          load_part8(part + prow * D + c8 + 8 * g, oj);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[8 * g + i] += wj * oj[i];
        }
      }
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  OutT* op = static_cast<OutT*>(a.o) + ci * a.chunk_elems + ((int64_t)row * a.H + h) * D + c8;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const float* ag = acc + 8 * g;
    if constexpr (sizeof(OutT) == 2) {
      bf16x8_t v;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (__bf16)(ag[i] * inv);
      *reinterpret_cast<bf16x8_t*>(op + 8 * g) = v;
    } else {
      f32x4_t v0 = {ag[0] * inv, ag[1] * inv, ag[2] * inv, ag[3] * inv};
      f32x4_t v1 = {ag[4] * inv, ag[5] * inv, ag[6] * inv, ag[7] * inv};
      *reinterpret_cast<f32x4_t*>(op + 8 * g) = v0;
      *reinterpret_cast<f32x4_t*>(op + 8 * g + 4) = v1;
    }
  }
  if (c8 == 0 && a.lse)
    a.lse[ci * a.chunk_lse + (int64_t)h * a.n + row] = (M == -INFINITY) ? M : M + logf(wsum);
}

// merge_lanes_kernel reads the bf16 path's fp16 partials, stored per wave as
// the attention kernel's lanes hold them: for the wave's 32 rows, 16-byte
// chunk c = 2 db + hf of lane l (values o[db][8 hf .. 8 hf + 7], i.e. dims
// 32 db + 16 hf + 4 (l / 32) + {0..3, 8..11} of row l % 32) at 16 (64 c + l)
// bytes from the wave's start, each row's values scaled by 2^-part_exp.
// One work group merges one 32-row slice of a unit: its threads read the
// chunks of every piece in order (consecutive threads, consecutive 16
// bytes; all of a thread's chunks belong to one row), combine them, and
// write the result out through LDS as whole rows.
// GROUPED: the units of a launch of groups (see UnitGroup).
template <int D, bool GROUPED>
__global__ __launch_bounds__(256) void merge_lanes_kernel(const MergeArgs a) {
  constexpr int NCH = 4 * D / 256;  // chunks per thread: a slice holds 4 D of them
  constexpr int RS = D + 8;         // LDS row stride (elements), off the bank period
  __shared__ __bf16 tile[32 * RS];
  const int slices = a.bm / 32;
  const int u = blockIdx.x / slices;
  const int sl = blockIdx.x - u * slices;
  const int64_t I = GROUPED ? a.iters : (int64_t)a.units * a.T;
  const int64_t w0 = first_wg_of(GROUPED ? unit_first_iter(a, u) : (int64_t)u * a.T, I, a.P);
  const int pieces = (int)(first_wg_of((GROUPED ? unit_first_iter(a, u + 1) : (int64_t)(u + 1) * a.T) - 1,
                                       I, a.P) -
                           w0 + 1);
  if (pieces <= 1) return;  // written whole by the attention kernel
  const int ci = u / a.upc, ul = u - ci * a.upc;  // chunk of a batched launch
  const int h = ul / a.QT, qt = ul - h * a.QT;
  const int row0 = qt * a.bm + sl * 32;  // the slice's first query row
  if (row0 >= a.n) return;
  const int t = threadIdx.x;
  const int lane = t & 63, r = lane & 31, hi = lane >> 5;
  const bool live = row0 + r < a.n;
  const int64_t slot0 =
      GROUPED ? part_slot_of(a, w0, u, I) : part_slot(w0, u, I, a.T, a.P, a.spw);
  // piece j >= 1 has the slot of its own (its range starts inside unit u)
  auto slot_of = [&](int j) -> int64_t { return j == 0 ? slot0 : (w0 + j) * a.spw; };
  const _Float16* part = reinterpret_cast<const _Float16*>(a.part_o);
  float M = -INFINITY, wsum = 0.f;
  float acc[8 * NCH];
#pragma unroll
  for (int i = 0; i < 8 * NCH; ++i) acc[i] = 0.f;
  if (live) {
    for (int j0 = 0; j0 < pieces; j0 += kMergeBatch) {
      // every load of a batch of pieces first, then the combination
      float lj[kMergeBatch];
      int ej[kMergeBatch];
      f16x8_t vj[kMergeBatch][NCH];
#pragma unroll
      for (int b = 0; b < kMergeBatch; ++b) {
        if (j0 + b < pieces) {
          const int64_t base = (slot_of(j0 + b) * a.bm + sl * 32);
          lj[b] = a.part_lse[base + r];
          ej[b] = a.part_exp[base + r];
#pragma unroll
          for (int k = 0; k < NCH; ++k)
            vj[b][k] = *reinterpret_cast<const f16x8_t*>(part + base * D + (t + 256 * k) * 8);
        }
      }
      float Mb = M;
#pragma unroll
      for (int b = 0; b < kMergeBatch; ++b)
        if (j0 + b < pieces) Mb = fmaxf(Mb, lj[b]);
      if (Mb == -INFINITY) continue;
      // rescale what earlier batches summed to the new maximum
      const float rs = (M == -INFINITY) ? 0.f : expf(M - Mb);
      wsum *= rs;
#pragma unroll
      for (int i = 0; i < 8 * NCH; ++i) acc[i] *= rs;
      M = Mb;
#pragma unroll
      for (int b = 0; b < kMergeBatch; ++b) {
        if (j0 + b < pieces) {
          const float wj = (lj[b] == -INFINITY) ? 0.f : expf(lj[b] - M);
          wsum += wj;
          const float ws = __builtin_amdgcn_ldexpf(wj, ej[b]);
#pragma unroll
          for (int k = 0; k < NCH; ++k)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[8 * k + i] += ws * (float)vj[b][k][i];
        }
      }
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  // the thread's values into the slice's rows in LDS (two runs of 4 dims per chunk)
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int c = (t >> 6) + 4 * k, db = c >> 1, hf = c & 1;
    const int d0 = 32 * db + 16 * hf + 4 * hi;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      f32x4_t v4 = {acc[8 * k + 4 * g], acc[8 * k + 4 * g + 1], acc[8 * k + 4 * g + 2],
                    acc[8 * k + 4 * g + 3]};
      v4 *= inv;
      *reinterpret_cast<bf16x4_t*>(&tile[r * RS + d0 + 8 * g]) = __builtin_convertvector(v4, bf16x4_t);
    }
  }
  if (t < 32 && live && a.lse)
    a.lse[ci * a.chunk_lse + (int64_t)h * a.n + row0 + r] = (M == -INFINITY) ? M : M + logf(wsum);
  __syncthreads();
  // whole rows out: 16 bytes per thread, D / 8 threads per row
  __bf16* ob = static_cast<__bf16*>(a.o) + ci * a.chunk_elems;
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int q = t + 256 * k, rr = q / (D / 8), c8 = q - rr * (D / 8);
    if (row0 + rr < a.n)
      *reinterpret_cast<bf16x8_t*>(ob + ((int64_t)(row0 + rr) * a.H + h) * D + 8 * c8) =
          *reinterpret_cast<const bf16x8_t*>(&tile[rr * RS + 8 * c8]);
  }
}

// ---------------------------------------------------------------------------
// Rotary position embedding of 8 consecutive elements (dims 8g .. 8g+7, four
// interleaved pairs) of a token at position pos: pair (2i, 2i+1) turns by the
// angle pos * base^(-2i/d), (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos).
// "Matrix-Game 4.0" (paper summary), experimental results: a RoPE fusion
// kernel; "WorldPlay2" (summary), inference optimisations: QKRoPE. The angle
// is formed and reduced in double precision (positions reach 10^5 and beyond,
// where an fp32 angle would be off by about 10^-2); the rotation is in fp32.

// Heads one thread of the rotary kernels turns with one set of angles.
constexpr int kRopeHeads = 4;

template <int D>
struct RopeAngles {
  float c[4], s[4];
};

// Inverse frequencies rope_base^(-2i/d), i = 0 .. d/2-1, in double, one per
// thread of the first d/2, into an LDS table shared by the work group.
template <int D>
__device__ __forceinline__ void rope_inv_freq(double* tab, double log2_base) {
  if (threadIdx.x < D / 2) tab[threadIdx.x] = exp2(-(2.0 * threadIdx.x / D) * log2_base);
  __syncthreads();
}

// Cosines and sines of the 4 pairs of dimension group g (dims 8g .. 8g+7) at
// position pos. They depend on neither the head nor Q/K, so the kernels take
// them once per (token, group) and turn several heads with them.
//
// Angles reach pos (10^5 and beyond) and are formed and reduced in double:
// theta = k pi/2 + x with |x| <= pi/4, x taken with three fused multiply-adds
// against pi/2 written as a sum of three doubles (Cody and Waite's additive
// reduction; with k below 2^20 the reduction error stays near 1e-16). The
// cosine and sine of x are then taken in fp32 (a few ulp of fp32, below the
// fp32 rotation's own rounding), and the quadrant k mod 4 swaps and negates
// them.
template <int D>
__device__ __forceinline__ RopeAngles<D> rope_angles(int g, int64_t pos, const double* inv_freq) {
  constexpr double kPio2Hi = 1.5707963267948966e+00;   // pi/2 rounded to double
  constexpr double kPio2Mid = 6.123233995736766e-17;   // pi/2 - kPio2Hi, rounded
  constexpr double kPio2Lo = -1.4973849048591698e-33;  // the remainder, rounded
  constexpr double k2OverPi = 6.3661977236758138e-01;
  RopeAngles<D> r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double theta = (double)pos * inv_freq[4 * g + j];
    const double k = rint(theta * k2OverPi);
    double x = fma(-k, kPio2Hi, theta);
    x = fma(-k, kPio2Mid, x);
    x = fma(-k, kPio2Lo, x);
    float sx, cx;
    sincosf((float)x, &sx, &cx);
    const int q = (int)((int64_t)k & 3);
    const float sq = (q & 1) ? cx : sx, cq = (q & 1) ? sx : cx;
    r.s[j] = (q & 2) ? -sq : sq;
    r.c[j] = ((q + 1) & 2) ? -cq : cq;
  }
  return r;
}

template <int D>
__device__ __forceinline__ void rope8(float (&x)[8], const RopeAngles<D>& r) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float c = r.c[j], s = r.s[j];
    const float x0 = x[2 * j], x1 = x[2 * j + 1];
    x[2 * j] = fmaf(x0, c, -(x1 * s));
    x[2 * j + 1] = fmaf(x0, s, x1 * c);
  }
}

// 8 elements of a bf16 (es 2) or fp32 (es 4) row as floats, and back (bf16
// rounded to nearest even).
__device__ __forceinline__ void load8(const char* p, int es, float (&x)[8]) {
  if (es == 2) {
    const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
  } else {
    const f32x4_t a = reinterpret_cast<const f32x4_t*>(p)[0];
    const f32x4_t b = reinterpret_cast<const f32x4_t*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
}
__device__ __forceinline__ void store8(char* p, int es, const float (&x)[8]) {
  if (es == 2) {
    bf16x8_t v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (__bf16)x[i];
    *reinterpret_cast<bf16x8_t*>(p) = v;
  } else {
    reinterpret_cast<f32x4_t*>(p)[0] = f32x4_t{x[0], x[1], x[2], x[3]};
    reinterpret_cast<f32x4_t*>(p)[1] = f32x4_t{x[4], x[5], x[6], x[7]};
  }
}

// Element offset of the destination block of an append: 0 when the host
// resolved the block, (id mod slots) * block_elems for a device-side chunk
// id, -1 (write nothing) for a negative one.
__device__ __forceinline__ int64_t append_block_offset(const AppendArgs& a) {
  if (!a.dev_chunk) return 0;
  const int64_t id = *a.dev_chunk;
  if (id < 0) return -1;
  return (id % a.slots) * a.block_elems;
}

// Fused K/V append: [n][H][d] -> the block's [H][n][d] rows (stride (S+R)*n*d
// between heads), converting to the cache dtype. blockIdx.y + kv0 selects K (0)
// or V (1). Each thread moves 8 elements. A rotated K goes through
// append_rope_k_kernel instead.
template <int D>
__global__ __launch_bounds__(256) void append_copy_kernel(const AppendArgs a, int es, int kv0) {
  constexpr int G = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.n * a.H * G;
  if (idx >= total) return;
  const int g = (int)(idx % G);
  const int64_t rh = idx / G;
  const int h = (int)(rh % a.H);
  const int r = (int)(rh / a.H);
  const bool isv = blockIdx.y + kv0 == 1;
  const int64_t blk = append_block_offset(a);
  if (blk < 0) return;
  const char* src = static_cast<const char*>(isv ? a.v : a.k) + (rh * D + g * 8) * es;
  char* dst = static_cast<char*>(isv ? a.vdst : a.kdst) +
              (blk + (int64_t)h * a.head_stride_elems + (int64_t)r * D + g * 8) * es;
  if (es == 2) {
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  } else {
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    uint4* d4 = reinterpret_cast<uint4*>(dst);
    d4[0] = s4[0];
    d4[1] = s4[1];
  }
}

// bf16 -> OCP e4m3 with the head's scale: code = round_to_nearest_even(x / s),
// saturated to +-448 (NaN stays NaN).
__device__ __forceinline__ uint2 e4m3x8(const float (&x)[8], float s) {
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = x[i] / s;
    y[i] = (fabsf(t) > 448.0f) ? copysignf(448.0f, t) : t;
  }
  int lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], lo, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], hi, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
  return make_uint2((unsigned)lo, (unsigned)hi);
}

// bf16 -> symmetric int8 with the head's scale: code = round_to_nearest_even(
// x / s) clamped to [-127, 127], NaN -> 0; byte i = element i.
__device__ __forceinline__ uint2 int8x8(const float (&x)[8], float s) {
  unsigned w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = x[i] / s;
    const float r = t == t ? fminf(fmaxf(__builtin_rintf(t), -127.0f), 127.0f) : 0.0f;
    w[i >> 2] |= ((unsigned)(int)r & 0xffu) << (8 * (i & 3));
  }
  return make_uint2(w[0], w[1]);
}

// Block index of an append's scales: host_blk, or (id mod slots) for a
// device-side chunk id (negative ids write nothing, as for the codes).
__device__ __forceinline__ int append_scale_block(const AppendArgs& a) {
  if (!a.dev_chunk) return a.host_blk;
  const int64_t id = *a.dev_chunk;
  return id < 0 ? -1 : (int)(id % a.slots);
}

// Scales of a per-block append (and of the current chunk's 8-bit copy): per
// head, scale = (largest |x| of the chunk's rows of that head) / 448 (/ 127
// for int8 K), 1 when that maximum is 0 or not finite (any NaN or infinity). One work group of 1024 threads per
// (head, K|V), each thread with up to 8 row loads in flight; blockIdx.y
// selects K (0) or V (1). ROPE (a rotary append): K's maximum is taken over
// the rotated rows, which are what the append stores.
template <int D, bool ROPE>
__global__ __launch_bounds__(1024) void append_amax_kernel(const AppendArgs a) {
  // fewer row loads in flight with rotation (its angles take registers)
  constexpr int G = D / 8, NT = 1024, U = ROPE ? 2 : 8;
  const int h = blockIdx.x;
  const bool isv = blockIdx.y == 1;
  const int bi = append_scale_block(a);
  if (bi < 0) return;
  __shared__ double inv_freq[ROPE ? D / 2 : 1];
  if constexpr (ROPE) rope_inv_freq<D>(inv_freq, a.rope_log2_base);
  const __bf16* src = static_cast<const __bf16*>(isv ? a.v : a.k);
  const int64_t total = (int64_t)a.n * G;
  float amax = 0.f;
  for (int64_t i0 = threadIdx.x; i0 < total; i0 += (int64_t)NT * U) {
    bf16x8_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + (int64_t)u * NT;
      const int64_t r = i / G, g = i % G;
      v[u] = i < total ? *reinterpret_cast<const bf16x8_t*>(src + (r * a.H + h) * D + 8 * g)
                       : bf16x8_t{};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (float)v[u][e];
      if (ROPE && !isv) {
        const int64_t i = i0 + (int64_t)u * NT;
        const int64_t r = i / G, g = i % G;
        rope8<D>(x, rope_angles<D>((int)g, a.rope_pos0 + r, inv_freq));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        // a NaN counts as an infinite magnitude: the maximum is then not
        // finite and the scale 1, as for an infinity
        amax = fmaxf(amax, x[e] == x[e] ? fabsf(x[e]) : INFINITY);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  __shared__ float wmax[NT / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = wmax[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) m = fmaxf(m, wmax[w]);
    const float qmax = (!isv && a.k_int8) ? 127.0f : 448.0f;
    const float sc = (m > 0.f && m <= 3.402823466e38f) ? m / qmax : 1.0f;
    (isv ? a.vsc : a.ksc)[(int64_t)bi * a.H + h] = sc;
  }
}

// The 8-bit append (e4m3, or int8 for the K of an INT8K_FP8V_BLOCK cache);
// blockIdx.y + kv0 selects K (0) or V (1).
template <int D>
__global__ __launch_bounds__(256) void append_fp8_kernel(const AppendArgs a, int kv0) {
  constexpr int G = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.n * a.H * G;
  if (idx >= total) return;
  const int g = (int)(idx % G);
  const int64_t rh = idx / G;
  const int h = (int)(rh % a.H);
  const int r = (int)(rh / a.H);
  const bool isv = blockIdx.y + kv0 == 1;
  const int64_t blk = append_block_offset(a);
  if (blk < 0) return;
  const float s = a.dev_scales
                      ? (isv ? a.vsc : a.ksc)[(int64_t)append_scale_block(a) * a.H + h]
                      : (isv ? a.v_scale[h] : a.k_scale[h]);
  float y[8];
  load8(reinterpret_cast<const char*>(static_cast<const __bf16*>(isv ? a.v : a.k) + rh * D +
                                      g * 8),
        2, y);
  unsigned char* dst = static_cast<unsigned char*>(isv ? a.vdst : a.kdst) +
                       (blk + (int64_t)h * a.head_stride_elems + (int64_t)r * D + g * 8);
  *reinterpret_cast<uint2*>(dst) = (!isv && a.k_int8) ? int8x8(y, s) : e4m3x8(y, s);
}

// Rotary embedding of the current chunk's Q (blockIdx.y 0) and K (1) into
// staging copies of the same [n][H][d] layout and dtype; token r at position
// pos0 + r. A thread owns one (token, 8-dim group), takes its cosines and sines
// once and turns that group in every head. The attention kernels then read the
// copies as q and k_cur.
template <int D>
__global__ __launch_bounds__(128) void rope_stage_kernel(const RopeStageArgs a, int es) {
  constexpr int G = D / 8;
  __shared__ double inv_freq[D / 2];
  rope_inv_freq<D>(inv_freq, a.log2_base);
  const int64_t idx = (int64_t)blockIdx.x * 128 + threadIdx.x;
  if (idx >= (int64_t)a.n * G) return;
  const int g = (int)(idx % G);
  const int r = (int)(idx / G);
  const RopeAngles<D> ang = rope_angles<D>(g, a.pos0 + r, inv_freq);
  const char* src = static_cast<const char*>(a.src[blockIdx.y]);
  char* dst = static_cast<char*>(a.dst[blockIdx.y]);
  const int h0 = blockIdx.z * kRopeHeads, h1 = min(a.H, h0 + kRopeHeads);
#pragma unroll
  for (int h = h0; h < h1; ++h) {
    const int64_t off = (((int64_t)r * a.H + h) * D + 8 * g) * es;
    float x[8];
    load8(src + off, es, x);
    rope8<D>(x, ang);
    store8(dst + off, es, x);
  }
}

// The rotated K of an append: like rope_stage_kernel (one thread per token,
// 8-dim group and kRopeHeads heads), writing the block's [H][n][d] rows in the cache
// dtype: bf16 or fp32 (es 2 or 4) when FP8 is false; when it is true, 8-bit
// codes with the head's scale (rotated first, in fp32, then quantised): e4m3,
// or int8 for the K of an INT8K_FP8V_BLOCK cache, with the per-head scale of
// the cache or the block's scale from the table append_amax_kernel fills.
template <int D, bool FP8>
__global__ __launch_bounds__(128) void append_rope_k_kernel(const AppendArgs a, int es) {
  constexpr int G = D / 8;
  __shared__ double inv_freq[D / 2];
  rope_inv_freq<D>(inv_freq, a.rope_log2_base);
  const int64_t idx = (int64_t)blockIdx.x * 128 + threadIdx.x;
  if (idx >= (int64_t)a.n * G) return;
  const int g = (int)(idx % G);
  const int r = (int)(idx / G);
  const RopeAngles<D> ang = rope_angles<D>(g, a.rope_pos0 + r, inv_freq);
  const int ies = FP8 ? 2 : es;
  const char* src = static_cast<const char*>(a.k);
  const int h0 = blockIdx.z * kRopeHeads, h1 = min(a.H, h0 + kRopeHeads);
#pragma unroll
  for (int h = h0; h < h1; ++h) {
    float x[8];
    load8(src + (((int64_t)r * a.H + h) * D + 8 * g) * ies, ies, x);
    rope8<D>(x, ang);
    const int64_t e = (int64_t)h * a.head_stride_elems + (int64_t)r * D + 8 * g;
    if constexpr (FP8) {
      const float sc =
          a.dev_scales ? a.ksc[(int64_t)append_scale_block(a) * a.H + h] : a.k_scale[h];
      *reinterpret_cast<uint2*>(static_cast<unsigned char*>(a.kdst) + e) =
          a.k_int8 ? int8x8(x, sc) : e4m3x8(x, sc);
    } else {
      store8(static_cast<char*>(a.kdst) + e * es, es, x);
    }
  }
}

template <int D>
int launch_attention_d(const Plan& p, const AttnArgs& a, hipStream_t s) {
  switch (p.kern) {
    case Kern::BF16:
      if (p.seq)
        hipLaunchKernelGGL((attn_bf16_kernel<D, true, false>), dim3(p.wgs), dim3(512), 0, s, a);
      else if (p.devt)
        hipLaunchKernelGGL((attn_bf16_kernel<D, false, true>), dim3(p.wgs), dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((attn_bf16_kernel<D, false, false>), dim3(p.wgs), dim3(512), 0, s, a);
      break;
    case Kern::FP8:
      if constexpr (D == 128) {
        // quantise the current chunk into the staging copy first, exactly as
        // appending it to the cache would
        AppendArgs q{};  // rope off: the chunk arrives already rotated when asked for
        q.k = a.kcur_in;
        q.v = a.vcur_in;
        q.kdst = const_cast<void*>(a.kcur);
        q.vdst = const_cast<void*>(a.vcur);
        q.head_stride_elems = (int64_t)a.n * D;
        q.n = a.n;
        q.H = a.H;
        for (int i = 0; i < kMaxHeadsFp8; ++i) {
          q.k_scale[i] = a.k_scale[i];
          q.v_scale[i] = a.v_scale[i];
        }
        if (a.blk) {
          // the chunk's own per-head scales, as an append would take them
          q.dev_scales = 1;
          q.k_int8 = a.i8k;
          q.host_blk = 0;
          q.ksc = const_cast<float*>(a.cur_sc);
          q.vsc = const_cast<float*>(a.cur_sc) + a.H;
          hipLaunchKernelGGL((append_amax_kernel<D, false>), dim3((unsigned)a.H, 2), dim3(1024), 0, s, q);
        }
        const int64_t total = (int64_t)a.n * a.H * (D / 8);
        hipLaunchKernelGGL(append_fp8_kernel<D>, dim3((unsigned)((total + 255) / 256), 2),
                           dim3(256), 0, s, q, 0);
        if (a.blk && a.i8k && p.devt)
          hipLaunchKernelGGL((attn_fp8_kernel<D, true, true, true>), dim3(p.wgs), dim3(512), 0,
                             s, a);
        else if (a.blk && a.i8k)
          hipLaunchKernelGGL((attn_fp8_kernel<D, true, false, true>), dim3(p.wgs), dim3(512), 0,
                             s, a);
        else if (a.blk && p.devt)
          hipLaunchKernelGGL((attn_fp8_kernel<D, true, true>), dim3(p.wgs), dim3(512), 0, s, a);
        else if (a.blk)
          hipLaunchKernelGGL((attn_fp8_kernel<D, true, false>), dim3(p.wgs), dim3(512), 0, s, a);
        else if (p.devt)
          hipLaunchKernelGGL((attn_fp8_kernel<D, false, true>), dim3(p.wgs), dim3(512), 0, s, a);
        else
          hipLaunchKernelGGL((attn_fp8_kernel<D, false, false>), dim3(p.wgs), dim3(512), 0, s, a);
      } else {
        return -1;
      }
      break;
    case Kern::F32:
      hipLaunchKernelGGL(attn_f32_kernel<D>, dim3(p.wgs), dim3(128), 0, s, a);
      break;
    default:
      return -1;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  if (p.merge) {
    MergeArgs m{};
    m.part_o = a.part_o;
    m.part_lse = a.part_lse;
    m.part_exp = a.part_exp;
    m.o = a.o;
    m.lse = a.lse;
    m.n = a.n;
    m.H = a.H;
    m.T = a.T;
    m.QT = a.QT;
    m.units = a.units;
    m.P = a.P;
    m.spw = a.spw;
    m.bm = p.bm;
    m.upc = a.upc;
    m.chunk_elems = a.chunk_elems;
    m.chunk_lse = a.chunk_lse;
    m.ngroups = a.ngroups;
    m.iters = a.iters;
    for (int g = 0; g < a.ngroups; ++g) m.grp[g] = a.grp[g];
    constexpr int RPB = 256 / (D / kMergeEpt);
    const int blocks = a.units * ((p.bm + RPB - 1) / RPB);
    if (p.kern == Kern::F32)
      hipLaunchKernelGGL((merge_kernel<D, float>), dim3(blocks), dim3(256), 0, s, m);
    else if (a.ngroups > 0)
      hipLaunchKernelGGL((merge_lanes_kernel<D, true>), dim3(a.units * (p.bm / 32)), dim3(256), 0,
                         s, m);
    else
      hipLaunchKernelGGL((merge_lanes_kernel<D, false>), dim3(a.units * (p.bm / 32)), dim3(256), 0,
                         s, m);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

}  // namespace

int launch_attention(const Plan& p, const AttnArgs& a, int head_dim, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 64) return launch_attention_d<64>(p, a, s);
  if (head_dim == 128) return launch_attention_d<128>(p, a, s);
  return -1;
}

int launch_rope_stage(bca_dtype dt, int head_dim, const RopeStageArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t total = (int64_t)a.n * (head_dim / 8);
  const dim3 grid((unsigned)((total + 127) / 128), 2, (unsigned)((a.H + kRopeHeads - 1) / kRopeHeads));
  const int es = dt == BCA_F32 ? 4 : 2;
  if (head_dim == 64)
    hipLaunchKernelGGL(rope_stage_kernel<64>, grid, dim3(128), 0, s, a, es);
  else if (head_dim == 128)
    hipLaunchKernelGGL(rope_stage_kernel<128>, grid, dim3(128), 0, s, a, es);
  else
    return -1;
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}

// Without rotation one launch moves K (blockIdx.y 0) and V (1). With it, V
// keeps that kernel (kv0 = 1, one grid row) and K goes through
// append_rope_k_kernel.
int launch_append(bca_dtype in, bca_dtype kv, int head_dim, const AppendArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t total = (int64_t)a.n * a.H * (head_dim / 8);
  const int kv0 = a.rope ? 1 : 0;
  const dim3 grid((unsigned)((total + 255) / 256), 2 - kv0);
  const dim3 rgrid((unsigned)(((int64_t)a.n * (head_dim / 8) + 127) / 128), 1,
                   (unsigned)((a.H + kRopeHeads - 1) / kRopeHeads));
  if (kv == BCA_FP8_E4M3 || kv == BCA_FP8_E4M3_BLOCK || kv == BCA_INT8K_FP8V_BLOCK) {
    if (head_dim != 128 || in != BCA_BF16) return -1;
    if (a.dev_scales && a.rope)
      hipLaunchKernelGGL((append_amax_kernel<128, true>), dim3((unsigned)a.H, 2), dim3(1024), 0, s,
                         a);
    else if (a.dev_scales)
      hipLaunchKernelGGL((append_amax_kernel<128, false>), dim3((unsigned)a.H, 2), dim3(1024), 0,
                         s, a);
    hipLaunchKernelGGL(append_fp8_kernel<128>, grid, dim3(256), 0, s, a, kv0);
    if (a.rope) hipLaunchKernelGGL((append_rope_k_kernel<128, true>), rgrid, dim3(128), 0, s, a, 1);
  } else {
    const int es = kv == BCA_F32 ? 4 : 2;
    if (head_dim == 64) {
      hipLaunchKernelGGL(append_copy_kernel<64>, grid, dim3(256), 0, s, a, es, kv0);
      if (a.rope)
        hipLaunchKernelGGL((append_rope_k_kernel<64, false>), rgrid, dim3(128), 0, s, a, es);
    } else {
      hipLaunchKernelGGL(append_copy_kernel<128>, grid, dim3(256), 0, s, a, es, kv0);
      if (a.rope)
        hipLaunchKernelGGL((append_rope_k_kernel<128, false>), rgrid, dim3(128), 0, s, a, es);
    }
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}

// The device-side chunk counter of a replayed chunk step: one thread adds 1.
__global__ void counter_advance_kernel(int64_t* counter) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *counter += 1;
}

int launch_counter_advance(int64_t* counter, void* stream) {
  hipLaunchKernelGGL(counter_advance_kernel, dim3(1), dim3(64), 0,
                     static_cast<hipStream_t>(stream), counter);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}

// Scratch of bca_attend_noalloc: device memory the library owns, for callers
// that cannot allocate. One copy per GPU the library runs on, held until the
// process ends. In host code `scratch` names a host-side stand-in, not device
// memory: the device address comes from hipGetSymbolAddress, looked up once
// per device (with that device current) and kept.
static __device__ __align__(256) unsigned char scratch[BCA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}

int device_compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return cus;
}

}  // namespace bca

// ---------------------------------------------------------------------------
// Measurement hooks (include/bca_probe.h; not part of the attention path): the
// matrix cores' dense bf16 and fp8 rates at the clock the chip runs at under load. Every wave issues
// v_mfma_f32_32x32x16_bf16 back to back into four independent accumulators;
// 8 waves per work group (two per SIMD), one work group per compute unit.
// The benchmark times the launch with events on the stream it runs on and
// reports the measured rate beside the published peak.
namespace bca {
namespace {

__global__ __launch_bounds__(512) void mfma_peak_kernel(float* out, int iters) {
  typedef __bf16 b8 __attribute__((ext_vector_type(8)));
  b8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f + 1e-3f * (float)((threadIdx.x + i) & 7));
    b[i] = (__bf16)(1.0f - 1e-3f * (float)((threadIdx.x * 3 + i) & 7));
  }
  f32x16_t acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
  for (int it = 0; it < iters; ++it) {
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc1, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc2, 0, 0, 0);
    acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += acc0[e] + acc1[e] + acc2[e] + acc3[e];
  // one value per wave reaches memory, so the products cannot be dropped
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * 8 + (threadIdx.x >> 6)] = s;
}

// The same with v_mfma_f32_32x32x64_f8f6f4 on e4m3 operands (the fp8 rate).
__global__ __launch_bounds__(512) void mfma_peak_fp8_kernel(float* out, int iters) {
  i32x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 + (int)((threadIdx.x + i) & 3);   // e4m3 values near 1
    b[i] = 0x38383838 + (int)((threadIdx.x * 3 + i) & 3);
  }
  f32x16_t acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
  for (int it = 0; it < iters; ++it) {
    acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc0, 0, 0, 0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc1, 0, 0, 0, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc2, 0, 0, 0, 0, 0, 0);
    acc3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc3, 0, 0, 0, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += acc0[e] + acc1[e] + acc2[e] + acc3[e];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * 8 + (threadIdx.x >> 6)] = s;
}

}  // namespace
}  // namespace bca

// FLOP of one probe launch: wgs * 8 waves * iters * 4 MFMAs * 32*32*16*2.
extern "C" double bca_probe_mfma_bf16_flops(int wgs, int iters) {
  return (double)wgs * 8.0 * (double)iters * 4.0 * 32768.0;
}

// FLOP of one fp8 probe launch: wgs * 8 waves * iters * 4 MFMAs * 32*32*64*2.
extern "C" double bca_probe_mfma_fp8_flops(int wgs, int iters) {
  return (double)wgs * 8.0 * (double)iters * 4.0 * 131072.0;
}

extern "C" int bca_probe_mfma_fp8(int wgs, int iters, float* out, void* stream) {
  if (wgs < 1 || iters < 1 || !out) return -1;
  hipLaunchKernelGGL(bca::mfma_peak_fp8_kernel, dim3((unsigned)wgs), dim3(512), 0,
                     static_cast<hipStream_t>(stream), out, iters);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}

// Launches the probe on `stream`; `out` is device memory of wgs * 8 floats.
extern "C" int bca_probe_mfma_bf16(int wgs, int iters, float* out, void* stream) {
  if (wgs < 1 || iters < 1 || !out) return -1;
  hipLaunchKernelGGL(bca::mfma_peak_kernel, dim3((unsigned)wgs), dim3(512), 0,
                     static_cast<hipStream_t>(stream), out, iters);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}
