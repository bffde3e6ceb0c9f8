/*
 * bca_oracle.c — CPU oracle for block-causal chunk attention over a chunk history.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline call this file. It shares no code, header, table or constant with
 * the GPU library, and the GPU library never calls it.
 *
 * Everything is plain C99 in double precision, written for a reader to check
 * against the pages by eye: an explicit dense 0/1 mask, scores only for the
 * keys the mask admits, and a two-pass softmax over the whole materialised row.
 * There is no ring buffer here: the history is every committed chunk, in id
 * order, and the mask alone decides what is visible.
 *
 * Sources:
 *  [WTF] "WanToFight: Real-Time Generative Game Engine for Multi-Player Combat
 *        Interaction" (xllm-io review): section 3 "model components" table,
 *        rows Block-Causal Attention (bidirectional inside a chunk; across
 *        chunks only the current one and the previous 2) and Rolling KV Cache;
 *        training Stage 2, causal adaptation (the dense mask is replaced by the
 *        block-causal one).
 *  [MG4] "Matrix-Game 4.0: Harnessing Video Models for Real-Time Playable Game
 *        Worlds" (paper summary): prerequisite "causal autoregression and KV
 *        cache" (recent window plus a reference frame; the window is split into
 *        intervals whose partial outputs are merged by log-sum-exp) and
 *        "technical novelty" (7 intervals, 8-bit K/V per interval).
 *  [RoPE] The pages name rotary position embedding only as a step fused into
 *        the path ("Matrix-Game 4.0" summary, experimental results: a RoPE
 *        fusion kernel; "WorldPlay2" summary, inference optimisations: QKRoPE).
 *        The reading here is the common one-dimensional rotary embedding with
 *        interleaved pairs (see bca_oracle_rope).
 *  [OCP] OCP 8-bit Floating Point Specification (OFP8), format E4M3: bias 7,
 *        no infinities, S.1111.111 is NaN, largest finite 448, subnormals
 *        m/8 * 2^-6. (External document: the pages only say "FP8".)
 *
 * Readings where the pages leave a step open are listed in the design notes;
 * the ones that shape this file:
 *  - visible history is chunk ids t-W .. t-1 (ids below 0 do not exist);
 *  - the current chunk is always visible and is passed separately;
 *  - the reference chunk, when used and present, is always visible and is not
 *    counted in W;
 *  - LSE is a natural logarithm; a row with no visible key (never produced by
 *    the block-causal mask, only by the split test's empty pieces) gets O = 0,
 *    LSE = -inf, and an -inf piece gets weight 0 in the merge.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_REF_ID ((int64_t)-2) /* marks the reference chunk in a key list */
#define ORACLE_CUR_ID ((int64_t)-3) /* marks the current chunk in a key list   */

/* Number of OpenMP threads the next parallel region would use (1 without OpenMP). */
int bca_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void bca_oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/*
 * Block-causal visibility of one key chunk for query chunk t [WTF model
 * components, Block-Causal Attention; MG4 prerequisite on the reference frame]:
 * the current chunk and the reference chunk are always visible (the reference
 * only if the caller asked for it: a reference block that was not requested
 * never enters the key list), a history chunk c is visible iff t-W <= c <= t-1.
 */
static int visible(int64_t c, int64_t t, int W) {
  if (c == ORACLE_CUR_ID || c == ORACLE_REF_ID) return 1;
  if (c < 0) return 0;
  return (c >= t - (int64_t)W) && (c <= t - 1);
}

/*
 * Attention of nq query rows over nk keys for H heads with an explicit dense
 * mask shared by all heads. Layouts: q [nq][H][d], k and v [nk][H][d],
 * mask [nq][nk] (1 = key admitted), o [nq][H][d], lse [H][nq].
 * For each head and row: s_j = scale * sum_k q_k k_jk for admitted j only
 * (masked keys are left out, never multiplied by zero), m = max_j s_j,
 * p_j = exp(s_j - m), l = sum_j p_j, O = sum_j p_j v_j / l, LSE = m + ln l.
 * literal != 0 skips the max subtraction (p_j = exp(s_j)); in double
 * precision both agree while |s| stays well below 700.
 */
int bca_oracle_attend_masked(int nq, int nk, int H, int d, const double* q, const double* k,
                             const double* v, const uint8_t* mask, double scale, int literal,
                             double* o, double* lse) {
  if (nq < 0 || nk < 0 || H < 1 || d < 1) return -1;
  long total = (long)H * nq;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 4)
  for (long hi = 0; hi < total; ++hi) {
    int h = (int)(hi / nq), i = (int)(hi % nq);
    double* s = (double*)malloc(sizeof(double) * (nk > 0 ? nk : 1));
    if (!s) {
      bad = 1;
      continue;
    }
    const double* qi = q + ((size_t)i * H + h) * d;
    const uint8_t* mi = mask + (size_t)i * nk;
    /* pass 1: scores of admitted keys and their maximum */
    double m = -INFINITY;
    int any = 0;
    for (int j = 0; j < nk; ++j) {
      if (!mi[j]) continue;
      const double* kj = k + ((size_t)j * H + h) * d;
      double acc = 0.0;
      for (int c = 0; c < d; ++c) acc += qi[c] * kj[c];
      s[j] = scale * acc;
      if (!any || s[j] > m) m = s[j];
      any = 1;
    }
    double* oi = o + ((size_t)i * H + h) * d;
    for (int c = 0; c < d; ++c) oi[c] = 0.0;
    if (!any) {
      lse[(size_t)h * nq + i] = -INFINITY;
      free(s);
      continue;
    }
    double shift = literal ? 0.0 : m;
    /* pass 2: weights, their sum and the weighted sum of values */
    double l = 0.0;
    for (int j = 0; j < nk; ++j) {
      if (!mi[j]) continue;
      double p = exp(s[j] - shift);
      l += p;
      const double* vj = v + ((size_t)j * H + h) * d;
      for (int c = 0; c < d; ++c) oi[c] += p * vj[c];
    }
    for (int c = 0; c < d; ++c) oi[c] /= l;
    lse[(size_t)h * nq + i] = shift + log(l);
    free(s);
  }
  return bad ? -2 : 0;
}

static int cmp_idx_by_id(const void* a, const void* b, const int64_t* ids) {
  int64_t x = ids[*(const int*)a], y = ids[*(const int*)b];
  return (x > y) - (x < y);
}

/* qsort has no context argument in C99: a small insertion sort keeps this plain. */
static void sort_by_id(int* idx, int count, const int64_t* ids) {
  for (int a = 1; a < count; ++a) {
    int cur = idx[a], b = a - 1;
    while (b >= 0 && cmp_idx_by_id(&idx[b], &cur, ids) > 0) {
      idx[b + 1] = idx[b];
      --b;
    }
    idx[b + 1] = cur;
  }
}

/*
 * Block-causal attention of query chunk t.
 *   hist_k, hist_v: [n_hist][n][H][d], chunk ids hist_ids[n_hist] (distinct, >= 0,
 *                   any order): every chunk committed so far, no ring.
 *   ref_k, ref_v:   [n][H][d] when has_ref, else ignored.
 *   q, k_cur, v_cur:[n][H][d]; o [n][H][d]; lse [H][n].
 * Steps:
 *   1. key list J = [reference (if use_ref and has_ref)] ++ [history in id order]
 *      ++ [current], with the chunk of every key recorded;
 *   2. dense mask M[i][j] = visible(chunk(j)) for every query row i, written
 *      out as an n x |J| byte matrix (the same for every row and head: the mask
 *      is block-causal, so every row of a chunk sees the same keys);
 *   3-4. bca_oracle_attend_masked (scores of admitted keys, two-pass softmax).
 * Returns 0, or a negative value on a bad argument.
 */
int bca_oracle_attend_rows(int H, int d, int n, int nq, int n_hist, const int64_t* hist_ids,
                           const double* hist_k, const double* hist_v, int has_ref,
                           const double* ref_k, const double* ref_v, const double* q,
                           const double* k_cur, const double* v_cur, int64_t t, int W,
                           int use_ref, double scale, int literal, double* o, double* lse);

int bca_oracle_attend(int H, int d, int n, int n_hist, const int64_t* hist_ids,
                      const double* hist_k, const double* hist_v, int has_ref,
                      const double* ref_k, const double* ref_v, const double* q,
                      const double* k_cur, const double* v_cur, int64_t t, int W, int use_ref,
                      double scale, int literal, double* o, double* lse) {
  return bca_oracle_attend_rows(H, d, n, n, n_hist, hist_ids, hist_k, hist_v, has_ref, ref_k,
                                ref_v, q, k_cur, v_cur, t, W, use_ref, scale, literal, o, lse);
}

/*
 * The same for nq query rows of chunk t (any subset of its n rows, q
 * [nq][H][d], o [nq][H][d], lse [H][nq]): every row of a chunk sees the same
 * keys, so the mask has nq identical rows.
 */
int bca_oracle_attend_rows(int H, int d, int n, int nq, int n_hist, const int64_t* hist_ids,
                           const double* hist_k, const double* hist_v, int has_ref,
                           const double* ref_k, const double* ref_v, const double* q,
                           const double* k_cur, const double* v_cur, int64_t t, int W,
                           int use_ref, double scale, int literal, double* o, double* lse) {
  if (H < 1 || d < 1 || n < 1 || nq < 1 || n_hist < 0 || W < 0 || t < 0) return -1;
  for (int a = 0; a < n_hist; ++a)
    if (hist_ids[a] < 0) return -1;
  int with_ref = (use_ref && has_ref) ? 1 : 0;
  int nblocks = with_ref + n_hist + 1;
  int nk = nblocks * n;
  size_t row = (size_t)H * d; /* elements per token */

  /* step 1: key list */
  int* order = (int*)malloc(sizeof(int) * (n_hist > 0 ? n_hist : 1));
  int64_t* block_id = (int64_t*)malloc(sizeof(int64_t) * nblocks);
  double* K = (double*)malloc(sizeof(double) * (size_t)nk * row);
  double* V = (double*)malloc(sizeof(double) * (size_t)nk * row);
  uint8_t* M = (uint8_t*)malloc((size_t)nq * nk);
  if (!order || !block_id || !K || !V || !M) {
    free(order), free(block_id), free(K), free(V), free(M);
    return -2;
  }
  for (int a = 0; a < n_hist; ++a) order[a] = a;
  sort_by_id(order, n_hist, hist_ids);
  int b = 0;
  size_t chunk = (size_t)n * row;
  if (with_ref) {
    memcpy(K + b * chunk, ref_k, sizeof(double) * chunk);
    memcpy(V + b * chunk, ref_v, sizeof(double) * chunk);
    block_id[b++] = ORACLE_REF_ID;
  }
  for (int a = 0; a < n_hist; ++a) {
    int src = order[a];
    memcpy(K + b * chunk, hist_k + (size_t)src * chunk, sizeof(double) * chunk);
    memcpy(V + b * chunk, hist_v + (size_t)src * chunk, sizeof(double) * chunk);
    block_id[b++] = hist_ids[src];
  }
  memcpy(K + b * chunk, k_cur, sizeof(double) * chunk);
  memcpy(V + b * chunk, v_cur, sizeof(double) * chunk);
  block_id[b++] = ORACLE_CUR_ID;

  /* step 2: the dense mask, one byte per (query row, key) */
  for (int i = 0; i < nq; ++i)
    for (int j = 0; j < nk; ++j) M[(size_t)i * nk + j] = (uint8_t)visible(block_id[j / n], t, W);

  /* steps 3-4 */
  int rc = bca_oracle_attend_masked(nq, nk, H, d, q, K, V, M, scale, literal, o, lse);
  free(order), free(block_id), free(K), free(V), free(M);
  return rc;
}

/*
 * Block-causal attention over a whole sequence at once, the training form
 * [WTF training Stage 2, causal adaptation: training uses the block-causal
 * mask itself], with a memory prefix of P context tokens ahead of chunk 0
 * that every chunk sees [MG4 prerequisite on the reference frame].
 *   q [C*n][H][d]; k, v [P + C*n][H][d] (prefix rows first); o [C*n][H][d];
 *   lse [H][C*n].
 * Query row i belongs to chunk i / n; key row j is a prefix token when j < P,
 * otherwise a token of chunk (j - P) / n. The dense mask, written out as a
 * (C*n) x (P + C*n) byte matrix, admits key j for row i iff j is a prefix
 * token, or its chunk c' satisfies chunk(i) - W <= c' <= chunk(i) (the chunk
 * itself, bidirectionally, and the W chunks before it). Then
 * bca_oracle_attend_masked.
 */
int bca_oracle_attend_sequence(int C, int n, int H, int d, int P, int W, const double* q,
                               const double* k, const double* v, double scale, double* o,
                               double* lse) {
  if (C < 1 || n < 1 || H < 1 || d < 1 || P < 0 || W < 0) return -1;
  int nq = C * n, nk = P + C * n;
  uint8_t* M = (uint8_t*)malloc((size_t)nq * nk);
  if (!M) return -2;
  for (int i = 0; i < nq; ++i) {
    int ci = i / n;
    for (int j = 0; j < nk; ++j) {
      int admit;
      if (j < P) {
        admit = 1;
      } else {
        int cj = (j - P) / n;
        admit = (cj >= ci - W) && (cj <= ci);
      }
      M[(size_t)i * nk + j] = (uint8_t)admit;
    }
  }
  int rc = bca_oracle_attend_masked(nq, nk, H, d, q, k, v, M, scale, 0, o, lse);
  free(M);
  return rc;
}

/*
 * Log-sum-exp merge of G partial results over disjoint key sets [MG4
 * prerequisite "causal autoregression and KV cache": partial outputs of the
 * window's intervals are merged by log-sum-exp]. Each partial is a normalised
 * attention output O_g with its LSE_g over its own keys.
 *   o_parts [G][rows][d], lse_parts [G][rows]  ->  o [rows][d], lse [rows]
 *   M = max_g LSE_g; w_g = exp(LSE_g - M), w_g = 0 when LSE_g = -inf;
 *   O = sum_g w_g O_g / sum_g w_g;  LSE = M + ln sum_g w_g.
 * Every row's sum_g w_g is a sum of exp over all keys, divided by exp(M),
 * so this equals one softmax over the union of the keys.
 */
int bca_oracle_lse_merge(int G, int rows, int d, const double* o_parts,
                         const double* lse_parts, double* o, double* lse) {
  if (G < 1 || rows < 0 || d < 1) return -1;
  for (int r = 0; r < rows; ++r) {
    double M = -INFINITY;
    for (int g = 0; g < G; ++g) {
      double x = lse_parts[(size_t)g * rows + r];
      if (x > M) M = x;
    }
    double* orow = o + (size_t)r * d;
    for (int c = 0; c < d; ++c) orow[c] = 0.0;
    if (M == -INFINITY) {
      lse[r] = -INFINITY;
      continue;
    }
    double wsum = 0.0;
    for (int g = 0; g < G; ++g) {
      double x = lse_parts[(size_t)g * rows + r];
      double w = (x == -INFINITY) ? 0.0 : exp(x - M);
      wsum += w;
      const double* op = o_parts + ((size_t)g * rows + r) * d;
      for (int c = 0; c < d; ++c) orow[c] += w * op[c];
    }
    for (int c = 0; c < d; ++c) orow[c] /= wsum;
    lse[r] = M + log(wsum);
  }
  return 0;
}

/*
 * OCP E4M3 decode [OCP]: sign s, exponent field e (4 bits), mantissa m (3 bits).
 *   e = 15 and m = 7: NaN;  e = 0: (-1)^s * m/8 * 2^-6;
 *   otherwise (-1)^s * (1 + m/8) * 2^(e-7).
 */
double bca_oracle_e4m3_decode(uint8_t code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

/*
 * OCP E4M3 encode of a float with round to nearest, ties to even, and
 * saturation: |x| at or beyond the largest finite value 448 (including
 * infinity) gives +-448; NaN gives 0x7F. The 127 non-negative finite codes
 * 0x00..0x7E are ordered by magnitude, so a binary search over their decoded
 * values finds the two neighbours of |x|; the nearer one is taken, and on an
 * exact tie the one with an even mantissa (code bit 0 clear). Zero keeps its
 * sign.
 */
static double e4m3_values[127];
static int e4m3_ready = 0;

static void e4m3_init(void) {
  if (e4m3_ready) return;
  for (int c = 0; c < 127; ++c) e4m3_values[c] = bca_oracle_e4m3_decode((uint8_t)c);
  e4m3_ready = 1;
}

uint8_t bca_oracle_e4m3_encode(float xf) {
  double x = (double)xf;
  if (x != x) return 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs(x);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  e4m3_init();
  /* largest code lo with value <= a */
  int lo = 0, hi = 126;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (e4m3_values[mid] <= a)
      lo = mid;
    else
      hi = mid - 1;
  }
  double vlo = e4m3_values[lo];
  if (vlo == a) return (uint8_t)(sign | lo);
  int up = lo + 1;
  double dlo = a - vlo, dup = e4m3_values[up] - a;
  int pick;
  if (dlo < dup)
    pick = lo;
  else if (dup < dlo)
    pick = up;
  else
    pick = (lo & 1) ? up : lo;
  return (uint8_t)(sign | pick);
}

/*
 * Quantisation of a cache chunk with one scale: code = encode(fp32(x / scale)),
 * the division done in single precision (the precision the GPU kernel uses to
 * decide the code, so both sides take the same decision).
 */
void bca_oracle_quant_e4m3(const float* x, long count, float scale, uint8_t* out) {
  e4m3_init();
#pragma omp parallel for schedule(static)
  for (long i = 0; i < count; ++i) {
    float y = x[i] / scale;
    out[i] = bca_oracle_e4m3_encode(y);
  }
}

/*
 * Per-interval scale of an 8-bit cache block [MG4 technical novelty: the
 * window is held as intervals of 8-bit K/V, and only the interval that
 * changed is re-quantised]. The pages fix neither the interval nor the rule;
 * the reading: an interval is one cache block (a chunk), and its scale per
 * head is the largest magnitude of the chunk's values in that head divided by
 * the largest code (448 for e4m3, 127 for int8), in single precision; 1 when
 * that maximum is 0 or not finite. x is [n][H][d] (fp32 values); out[H].
 */
void bca_oracle_block_scales(const float* x, int n, int H, int d, float qmax, float* out) {
  for (int h = 0; h < H; ++h) {
    float a = 0.0f;
    for (int r = 0; r < n; ++r)
      for (int j = 0; j < d; ++j) {
        float v = fabsf(x[((size_t)r * H + h) * d + j]);
        if (v > a || v != v) a = v;
      }
    out[h] = (a > 0.0f && a <= FLT_MAX) ? a / qmax : 1.0f;
  }
}

/*
 * Symmetric int8 code of a value with one scale [MG4 technical novelty: INT8
 * keys]: code = round to nearest even of fp32(x / scale), clamped to
 * [-127, 127] (the code -128 is never produced, so the range is symmetric);
 * NaN gives 0. The value a code stands for is code * scale.
 */
void bca_oracle_quant_int8(const float* x, long count, float scale, int8_t* out) {
#pragma omp parallel for schedule(static)
  for (long i = 0; i < count; ++i) {
    float y = x[i] / scale;
    if (y != y) {
      out[i] = 0;
      continue;
    }
    if (y > 127.0f) y = 127.0f;
    if (y < -127.0f) y = -127.0f;
    /* round half to even, written out: nearest integer below, then compare
       the remainder with one half */
    double f = floor((double)y), rem = (double)y - f;
    long q = (long)f;
    if (rem > 0.5 || (rem == 0.5 && (q & 1))) q += 1;
    out[i] = (int8_t)q;
  }
}

/*
 * Rotary position embedding of one chunk's vectors [RoPE]. x and y are
 * [n][H][d] (d even); token r of the chunk has position pos0 + r. Each pair of
 * dimensions (2i, 2i+1), i = 0 .. d/2 - 1, is rotated by the angle
 *     theta = position * base^(-2i/d)
 * as (x0, x1) -> (x0 cos theta - x1 sin theta, x0 sin theta + x1 cos theta),
 * the same for every head. Position 0 leaves x unchanged, lengths are kept,
 * and the inner product of a query at position m with a key at position k
 * depends on m - k only. Returns 0, or -1 for an invalid argument.
 */
int bca_oracle_rope(int n, int H, int d, const double* x, int64_t pos0, double base, double* y) {
  if (n < 0 || H < 1 || d < 2 || (d & 1) || !(base > 0.0)) return -1;
  for (int r = 0; r < n; ++r) {
    const double pos = (double)(pos0 + r);
    for (int h = 0; h < H; ++h) {
      const double* xi = x + ((size_t)r * H + h) * d;
      double* yi = y + ((size_t)r * H + h) * d;
      for (int i = 0; i < d / 2; ++i) {
        const double theta = pos * pow(base, -2.0 * i / d);
        const double c = cos(theta), s = sin(theta);
        const double x0 = xi[2 * i], x1 = xi[2 * i + 1];
        yi[2 * i] = x0 * c - x1 * s;
        yi[2 * i + 1] = x0 * s + x1 * c;
      }
    }
  }
  return 0;
}
