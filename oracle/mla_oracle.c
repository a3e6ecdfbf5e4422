/*
 * mla_oracle.c -- CPU oracle for paged MLA decode with split-KV.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, link or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with the
 * HIP library; both sides only share the seeded input generator.
 *
 * Plain, slow, obviously correct.  Inputs are bf16 or fp16 bit patterns
 * (widened to double exactly); every sum, exp and log is done in double
 * precision.
 *
 * What is computed (sources: the pages on FlashMLA):
 *   - "DeepSeek 开源记-第1天-FlashMLA" (cnblogs), section 2 "核心功能": head
 *     dim is fixed at 576, value dim at 512, Shared-KV mode (the value is the
 *     leading part of the same cached row), an efficient softmax;
 *     section 4 "核心实现": blockwise scores, softmax, merge of partial
 *     outputs; section 6 "使用方法": the two calls and their arguments
 *     (cache_seqlens, s_q*h_q//h_kv, h_kv, q, blocked_k, block_table, dv,
 *     tile_scheduler_metadata, num_splits, causal) and the (output, lse) pair.
 *   - "DeepSeek代碼開源第一彈Flash MLA" (ygpos news): BF16, paged KV cache with
 *     block size 64, variable-length sequences.
 *   - "DeepSeek 开源记-第1天-FlashMLA" (cnblogs), section 2 "核心功能": FP16
 *     beside BF16 (the other pages name BF16 only; the jsxs2 explainer's
 *     section 2.1 says BF16 only).
 *   - FlashMLA explainer (jsxs2.com), section 3.1 "分块调度与并行计算": the work
 *     is cut into small blocks that run in parallel (the split scheduler).
 *
 * Readings where the pages are silent (each is also listed in the design doc):
 *   - the softmax scale multiplies the scores before exp, and lse includes it;
 *   - lse is the natural log of the softmax denominator, one per (b, t, h);
 *   - causal: the s_q query tokens are the last s_q positions of the
 *     sequence, so query t sees keys j <= N - s_q + t;
 *   - a row with no visible key has out = 0 and lse = -inf;
 *   - KV head g serves query heads h with h / (h_q / h_kv) == g;
 *   - cache rows past N in the last page and block_table entries past
 *     ceil(N / page) are not part of the sequence and are never read.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_PAGE (-2)
#define ORACLE_ERR_NOMEM (-3)

#define ORACLE_BF16 0
#define ORACLE_FP16 1

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_to_double(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exponent 0 holds zero and the subnormals f * 2^-24; exponent 31
 * holds infinities (f = 0) and NaNs.  Every value is exact in double. */
static double fp16_to_double(uint16_t bits) {
  const int sign = bits >> 15, e = (bits >> 10) & 31, f = bits & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  return sign ? -v : v;
}

static double widen(uint16_t bits, int dtype) {
  return dtype == ORACLE_FP16 ? fp16_to_double(bits) : bf16_to_double(bits);
}

/* Widen n bit patterns of the given type (0 bf16, 1 fp16) to double. */
int mla_oracle_widen(const uint16_t *bits, long n, int dtype, double *out) {
  if (!bits || !out || n < 0 || (dtype != ORACLE_BF16 && dtype != ORACLE_FP16)) return ORACLE_ERR_ARG;
  for (long i = 0; i < n; ++i) out[i] = widen(bits[i], dtype);
  return ORACLE_OK;
}

int mla_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Number of keys that query token t of sequence b may attend to. */
static long visible_keys(long n, int s_q, int t, int causal) {
  long l = causal ? n - s_q + t + 1 : n;
  if (l > n) l = n;
  if (l < 0) l = 0;
  return l;
}

/* Pointer to the cached 576-wide row of logical key j of sequence b, KV head g,
 * found through the block table (paged cache, page = page_size tokens). */
static const uint16_t *key_row(const uint16_t *kcache, const int32_t *block_table, int b, long j,
                               int g, int h_kv, int d, int page_size, int max_blocks) {
  long page = block_table[(long)b * max_blocks + j / page_size];
  long slot = j % page_size;
  return kcache + ((page * page_size + slot) * h_kv + g) * (long)d;
}

static int check_args(const int32_t *block_table, const int32_t *seqlens, int B, int s_q, int h_q,
                      int h_kv, int d, int dv, int page_size, int num_pages, int max_blocks) {
  if (B < 0 || s_q < 1 || h_q < 1 || h_kv < 1 || h_q % h_kv != 0 || d < 1 || dv < 1 || dv > d ||
      page_size < 1 || num_pages < 0 || max_blocks < 0)
    return ORACLE_ERR_ARG;
  for (int b = 0; b < B; ++b) {
    long n = seqlens[b];
    if (n < 0) return ORACLE_ERR_ARG;
    long need = (n + page_size - 1) / page_size;
    if (need > max_blocks) return ORACLE_ERR_ARG;
    for (long i = 0; i < need; ++i) {
      int32_t p = block_table[(long)b * max_blocks + i];
      if (p < 0 || p >= num_pages) return ORACLE_ERR_PAGE;
    }
  }
  return ORACLE_OK;
}

/* Scaled score of every key j in [0, n_keys) for one query row. */
static void row_scores(const uint16_t *qrow, const uint16_t *kcache, const int32_t *block_table,
                       int b, int g, long n_keys, int h_kv, int d, int page_size, int max_blocks,
                       double scale, int dtype, double *s) {
  for (long j = 0; j < n_keys; ++j) {
    const uint16_t *k = key_row(kcache, block_table, b, j, g, h_kv, d, page_size, max_blocks);
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += widen(qrow[c], dtype) * widen(k[c], dtype);
    s[j] = scale * acc;
  }
}

/* Softmax attention of one row over keys [j0, j1): lse of the piece and
 * out = sum_j exp(s_j - lse) * V_j, V_j = first dv entries of key row j.
 * An empty piece gives lse = -inf and out = 0. */
static void attend_range(const double *s, long j0, long j1, const uint16_t *kcache,
                         const int32_t *block_table, int b, int g, int h_kv, int d, int dv,
                         int page_size, int max_blocks, int dtype, double *out, double *lse) {
  for (int v = 0; v < dv; ++v) out[v] = 0.0;
  if (j1 <= j0) {
    *lse = -INFINITY;
    return;
  }
  double m = -INFINITY;
  for (long j = j0; j < j1; ++j)
    if (s[j] > m) m = s[j];
  double denom = 0.0;
  for (long j = j0; j < j1; ++j) denom += exp(s[j] - m);
  double l = m + log(denom);
  for (long j = j0; j < j1; ++j) {
    double w = exp(s[j] - l);
    const uint16_t *k = key_row(kcache, block_table, b, j, g, h_kv, d, page_size, max_blocks);
    for (int v = 0; v < dv; ++v) out[v] += w * widen(k[v], dtype);
  }
  *lse = l;
}

/*
 * Reference decode.  Layouts (row-major, 16-bit bit patterns as uint16 of
 * type dtype: 0 bf16, 1 fp16):
 *   q           [B, s_q, h_q, d]
 *   kcache      [num_pages, page_size, h_kv, d]
 *   block_table [B, max_blocks]   physical page of logical block i of sequence b
 *   seqlens     [B]
 *   out         [B, s_q, h_q, dv]  (double)
 *   lse         [B, s_q, h_q]      (double, natural log)
 * Returns 0, or a negative code for bad arguments / out-of-range pages.
 */
int mla_oracle_decode(const uint16_t *q, const uint16_t *kcache, const int32_t *block_table,
                      const int32_t *seqlens, int B, int s_q, int h_q, int h_kv, int d, int dv,
                      int page_size, int num_pages, int max_blocks, int causal, double scale,
                      int dtype, double *out, double *lse) {
  if (dtype != ORACLE_BF16 && dtype != ORACLE_FP16) return ORACLE_ERR_ARG;
  int rc = check_args(block_table, seqlens, B, s_q, h_q, h_kv, d, dv, page_size, num_pages,
                      max_blocks);
  if (rc != ORACLE_OK) return rc;
  long rows = (long)B * s_q * h_q;
  int heads_per_group = h_q / h_kv;
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long r = 0; r < rows; ++r) {
    int h = (int)(r % h_q);
    int t = (int)((r / h_q) % s_q);
    int b = (int)(r / ((long)h_q * s_q));
    int g = h / heads_per_group;
    long n_vis = visible_keys(seqlens[b], s_q, t, causal);
    double *s = (double *)malloc(sizeof(double) * (size_t)(n_vis > 0 ? n_vis : 1));
    if (!s) {
#pragma omp atomic write
      failed = 1;
      continue;
    }
    row_scores(q + r * d, kcache, block_table, b, g, n_vis, h_kv, d, page_size, max_blocks, scale,
               dtype, s);
    attend_range(s, 0, n_vis, kcache, block_table, b, g, h_kv, d, dv, page_size, max_blocks,
                 dtype, out + r * dv, lse + r);
    free(s);
  }
  return failed ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/*
 * Split-KV model of the decode (the pages' "output merge" step).  Sequence b's
 * key positions are cut at cuts[cut_ptr[b] .. cut_ptr[b+1]) (ascending token
 * indices strictly inside (0, N)); every piece is attended on its own,
 * giving (o_k, lse_k), and the pieces are merged by their log-sum-exp:
 *   lse = ln sum_k exp(lse_k),   out = sum_k exp(lse_k - lse) * o_k.
 * Pieces with no visible key carry lse_k = -inf and weigh nothing.
 */
int mla_oracle_decode_split(const uint16_t *q, const uint16_t *kcache, const int32_t *block_table,
                            const int32_t *seqlens, int B, int s_q, int h_q, int h_kv, int d,
                            int dv, int page_size, int num_pages, int max_blocks, int causal,
                            double scale, int dtype, const int32_t *cut_ptr, const int32_t *cuts,
                            double *out, double *lse) {
  if (dtype != ORACLE_BF16 && dtype != ORACLE_FP16) return ORACLE_ERR_ARG;
  int rc = check_args(block_table, seqlens, B, s_q, h_q, h_kv, d, dv, page_size, num_pages,
                      max_blocks);
  if (rc != ORACLE_OK) return rc;
  for (int b = 0; b < B; ++b) {
    if (cut_ptr[b + 1] < cut_ptr[b]) return ORACLE_ERR_ARG;
    int prev = 0;
    for (int i = cut_ptr[b]; i < cut_ptr[b + 1]; ++i) {
      if (cuts[i] <= prev || cuts[i] >= seqlens[b]) return ORACLE_ERR_ARG;
      prev = cuts[i];
    }
  }
  long rows = (long)B * s_q * h_q;
  int heads_per_group = h_q / h_kv;
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long r = 0; r < rows; ++r) {
    int h = (int)(r % h_q);
    int t = (int)((r / h_q) % s_q);
    int b = (int)(r / ((long)h_q * s_q));
    int g = h / heads_per_group;
    long n_vis = visible_keys(seqlens[b], s_q, t, causal);
    int n_pieces = cut_ptr[b + 1] - cut_ptr[b] + 1;
    double *s = (double *)malloc(sizeof(double) * (size_t)(n_vis > 0 ? n_vis : 1));
    double *o_k = (double *)malloc(sizeof(double) * (size_t)dv * n_pieces);
    double *lse_k = (double *)malloc(sizeof(double) * (size_t)n_pieces);
    if (!s || !o_k || !lse_k) {
      free(s);
      free(o_k);
      free(lse_k);
#pragma omp atomic write
      failed = 1;
      continue;
    }
    row_scores(q + r * d, kcache, block_table, b, g, n_vis, h_kv, d, page_size, max_blocks, scale,
               dtype, s);
    for (int k = 0; k < n_pieces; ++k) {
      long j0 = (k == 0) ? 0 : cuts[cut_ptr[b] + k - 1];
      long j1 = (k == n_pieces - 1) ? seqlens[b] : cuts[cut_ptr[b] + k];
      if (j1 > n_vis) j1 = n_vis;
      if (j0 > j1) j0 = j1;
      attend_range(s, j0, j1, kcache, block_table, b, g, h_kv, d, dv, page_size, max_blocks,
                   dtype, o_k + (long)k * dv, lse_k + k);
    }
    /* merge */
    double m = -INFINITY;
    for (int k = 0; k < n_pieces; ++k)
      if (lse_k[k] > m) m = lse_k[k];
    double *o = out + r * dv;
    for (int v = 0; v < dv; ++v) o[v] = 0.0;
    if (m == -INFINITY) {
      lse[r] = -INFINITY;
    } else {
      double acc = 0.0;
      for (int k = 0; k < n_pieces; ++k) acc += exp(lse_k[k] - m);
      double l = m + log(acc);
      for (int k = 0; k < n_pieces; ++k) {
        double w = exp(lse_k[k] - l);
        for (int v = 0; v < dv; ++v) o[v] += w * o_k[(long)k * dv + v];
      }
      lse[r] = l;
    }
    free(s);
    free(o_k);
    free(lse_k);
  }
  return failed ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/*
 * Split-KV tile scheduling (the pages' block scheduling: the work is cut into
 * small blocks run in parallel, and get_mla_metadata returns
 * tile_scheduler_metadata and num_splits from cache_seqlens).  The pages give
 * no rule; this is the rule the library documents, written out step by step.
 * A "unit" is unit_tokens consecutive keys of one sequence; f = fixed_cost.
 *
 *   1. U_b = ceil(N_b / unit_tokens) units.  On a cost line counted in half
 *      units, sequence b occupies 2 U_b + 2 f positions: f for its start-up
 *      work, two per unit, f for its finishing work (one fixed cost of f
 *      units per sequence, half at each end).
 *   2. S_b = sum over b' < b of (2 U_b' + 2 f); TOT = S_B.  The parts
 *      share the line evenly: position x belongs to part
 *      floor(x num_parts / TOT), so part p spans positions
 *      [ceil(p TOT / num_parts), ceil((p + 1) TOT / num_parts)).  When
 *      TOT < 2 num_parts every part spans 2 positions instead (part
 *      floor(x / 2)).  (At least 2 positions per part put a unit midpoint
 *      into every part that lies inside a sequence's units, so the pieces of
 *      a sequence sit in consecutive parts.)
 *   3. Unit i of sequence b is placed at its midpoint, x = S_b + f + 2 i + 1,
 *      and belongs to that position's part.  A sequence with no unit gets
 *      one empty piece in the part of x = S_b + f.
 *   4. A piece is the run of one sequence's units inside one part; pieces of
 *      a sequence sit in consecutive parts.  num_splits[b+1] - num_splits[b]
 *      is the number of pieces of sequence b (num_splits[0] = 0).
 *   5. Per part p, 8 int32 words: first sequence bb, first key of its
 *      piece, last sequence be, end key (exclusive, at most N) of its piece,
 *      the partial slot of bb's piece (num_splits[bb] + its split index),
 *      N_bb, N_be, and num_splits[be] (the partial slot of be's piece, whose
 *      split index is 0).  A part with no piece stores first = 0, last = -1
 *      and zeros elsewhere.
 * Every unit is visited one by one here (no closed form), so the result pins
 * a scheduler that computes piece bounds arithmetically.
 */

/* The part of cost position x (step 2 above). */
static long part_of(long x, long tot, long parts) {
  return tot < 2 * parts ? x / 2 : x * parts / tot;
}

int mla_oracle_schedule(const int32_t *seqlens, int B, int unit_tokens, int num_parts,
                        int fixed_cost, int32_t *tile_meta, int32_t *num_splits) {
  if (B < 0 || unit_tokens < 1 || num_parts < 1 || fixed_cost < 1) return ORACLE_ERR_ARG;
  for (int b = 0; b < B; ++b)
    if (seqlens[b] < 0) return ORACLE_ERR_ARG;
  for (long i = 0; i < (long)num_parts * 8; ++i) tile_meta[i] = 0;
  for (int p = 0; p < num_parts; ++p) tile_meta[(long)p * 8 + 2] = -1; /* empty until a piece lands */
  if (B == 0) {
    num_splits[0] = 0;
    return ORACLE_OK;
  }
  const long f = fixed_cost;
  long tot = 0;
  for (int b = 0; b < B; ++b) tot += 2 * (((long)seqlens[b] + unit_tokens - 1) / unit_tokens) + 2 * f;
  const long P = num_parts;

  /* Walk every unit in order; each change of part (or of sequence) starts a
   * new piece.  For every piece remember its sequence, part, split index and
   * key range; then fill the per-part words from the pieces. */
  long S = 0;
  int pieces = 0;
  num_splits[0] = 0;
  for (int b = 0; b < B; ++b) {
    const long n = seqlens[b];
    const long u = (n + unit_tokens - 1) / unit_tokens;
    int split = 0;
    if (u == 0) {
      const long p = part_of(S + f, tot, P);
      int32_t *w = tile_meta + p * 8;
      if (w[2] < 0) { /* the part's first piece */
        w[0] = b;
        w[1] = 0;
        w[4] = pieces;
        w[5] = (int32_t)n;
      }
      w[2] = b;
      w[3] = 0;
      w[6] = (int32_t)n;
      ++pieces;
      split = 1;
    } else {
      long cur = -1;
      for (long i = 0; i < u; ++i) {
        const long p = part_of(S + f + 2 * i + 1, tot, P);
        const long key_lo = i * unit_tokens;
        const long key_hi = (i + 1) * unit_tokens < n ? (i + 1) * unit_tokens : n;
        int32_t *w = tile_meta + p * 8;
        if (p != cur) { /* a new piece of sequence b in part p */
          cur = p;
          if (w[2] < 0) { /* and the part's first piece */
            w[0] = b;
            w[1] = (int32_t)key_lo;
            w[4] = pieces;
            w[5] = (int32_t)n;
          }
          w[2] = b;
          w[6] = (int32_t)n;
          ++pieces;
          ++split;
        }
        w[3] = (int32_t)key_hi;
      }
    }
    num_splits[b + 1] = num_splits[b] + split;
    S += 2 * u + 2 * f;
  }
  /* word 7: num_splits[be], known once every sequence is walked */
  for (int p = 0; p < num_parts; ++p) {
    int32_t *w = tile_meta + (long)p * 8;
    if (w[2] >= 0) w[7] = num_splits[w[2]];
  }
  return ORACLE_OK;
}
