/*
 * Sanitizer harness for the CPU oracle (test infrastructure): built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py
 * and run on small inputs that reach every branch of the oracle: empty and
 * one-key sequences, a last page that is partly used, causal rows with no
 * visible key, several KV heads, both element types, split cut points, the
 * scheduler with empty sequences and more parts than units, and the argument
 * checks.  A sanitizer report or a wrong status code fails the run.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int mla_oracle_widen(const uint16_t *bits, long n, int dtype, double *out);
int mla_oracle_decode(const uint16_t *q, const uint16_t *kcache, const int32_t *block_table,
                      const int32_t *seqlens, int B, int s_q, int h_q, int h_kv, int d, int dv,
                      int page_size, int num_pages, int max_blocks, int causal, double scale,
                      int dtype, double *out, double *lse);
int mla_oracle_decode_split(const uint16_t *q, const uint16_t *kcache, const int32_t *block_table,
                            const int32_t *seqlens, int B, int s_q, int h_q, int h_kv, int d,
                            int dv, int page_size, int num_pages, int max_blocks, int causal,
                            double scale, int dtype, const int32_t *cut_ptr, const int32_t *cuts,
                            double *out, double *lse);
int mla_oracle_schedule(const int32_t *seqlens, int B, int unit_tokens, int num_parts,
                        int fixed_cost, int32_t *tile_meta, int32_t *num_splits);

static int failures = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                 \
    }                                                             \
  } while (0)

static uint32_t rng_state = 12345u;
static uint16_t rand_bits(void) {
  /* small finite values of either type: sign, exponent near 1, random mantissa */
  rng_state = rng_state * 1664525u + 1013904223u;
  return (uint16_t)(0x3c00u | ((rng_state >> 9) & 0x03ffu) | ((rng_state >> 16) & 0x8000u));
}

int main(void) {
  enum { D = 24, DV = 16, PAGE = 4, H_KV = 2, H_Q = 4, S_Q = 3, B = 5, MAXB = 4, PAGES = 16 };
  const int32_t seqlens[B] = {0, 1, 5, 16, 2};
  int32_t table[B * MAXB];
  for (int i = 0; i < B * MAXB; ++i) table[i] = (i * 7) % PAGES;
  uint16_t *q = malloc(sizeof(uint16_t) * B * S_Q * H_Q * D);
  uint16_t *kc = malloc(sizeof(uint16_t) * PAGES * PAGE * H_KV * D);
  double *out = malloc(sizeof(double) * B * S_Q * H_Q * DV);
  double *lse = malloc(sizeof(double) * B * S_Q * H_Q);
  double *out2 = malloc(sizeof(double) * B * S_Q * H_Q * DV);
  double *lse2 = malloc(sizeof(double) * B * S_Q * H_Q);
  if (!q || !kc || !out || !lse || !out2 || !lse2) return 2;
  for (int i = 0; i < B * S_Q * H_Q * D; ++i) q[i] = rand_bits();
  for (int i = 0; i < PAGES * PAGE * H_KV * D; ++i) kc[i] = rand_bits();

  double w[4];
  const uint16_t bits[4] = {0x3f80, 0x0001, 0x7c00, 0xfc00};
  EXPECT(mla_oracle_widen(bits, 4, 0, w) == 0);
  EXPECT(mla_oracle_widen(bits, 4, 1, w) == 0 && isinf(w[2]) && w[3] < 0);
  EXPECT(mla_oracle_widen(bits, 4, 2, w) != 0);

  for (int dtype = 0; dtype < 2; ++dtype) {
    for (int causal = 0; causal < 2; ++causal) {
      EXPECT(mla_oracle_decode(q, kc, table, seqlens, B, S_Q, H_Q, H_KV, D, DV, PAGE, PAGES, MAXB,
                               causal, 0.2, dtype, out, lse) == 0);
      /* empty sequence: out 0, lse -inf; causal rows of the 1- and 2-key
       * sequences see no key for the first tokens */
      EXPECT(isinf(lse[0]) && lse[0] < 0 && out[0] == 0.0);
      const int32_t cut_ptr[B + 1] = {0, 0, 0, 2, 5, 5};
      const int32_t cuts[5] = {1, 3, 4, 9, 15};
      EXPECT(mla_oracle_decode_split(q, kc, table, seqlens, B, S_Q, H_Q, H_KV, D, DV, PAGE, PAGES,
                                     MAXB, causal, 0.2, dtype, cut_ptr, cuts, out2, lse2) == 0);
      double worst = 0.0;
      for (int i = 0; i < B * S_Q * H_Q; ++i) {
        if (isinf(lse[i])) {
          EXPECT(isinf(lse2[i]));
          continue;
        }
        worst = fmax(worst, fabs(lse[i] - lse2[i]));
        for (int v = 0; v < DV; ++v) worst = fmax(worst, fabs(out[i * DV + v] - out2[i * DV + v]));
      }
      EXPECT(worst < 1e-12);
    }
  }
  /* argument checks */
  const int32_t bad_len[B] = {0, 1, 5, 17, 2}; /* needs 5 blocks > MAXB */
  EXPECT(mla_oracle_decode(q, kc, table, bad_len, B, S_Q, H_Q, H_KV, D, DV, PAGE, PAGES, MAXB, 0,
                           0.2, 0, out, lse) != 0);
  int32_t bad_table[B * MAXB];
  for (int i = 0; i < B * MAXB; ++i) bad_table[i] = table[i];
  bad_table[2 * MAXB + 1] = PAGES; /* out of the pool, inside sequence 2's pages */
  EXPECT(mla_oracle_decode(q, kc, bad_table, seqlens, B, S_Q, H_Q, H_KV, D, DV, PAGE, PAGES, MAXB,
                           0, 0.2, 0, out, lse) != 0);
  EXPECT(mla_oracle_decode(q, kc, table, seqlens, B, S_Q, H_Q, 3, D, DV, PAGE, PAGES, MAXB, 0, 0.2,
                           0, out, lse) != 0);
  const int32_t bad_ptr[B + 1] = {0, 0, 0, 1, 1, 1};
  const int32_t bad_cut[1] = {5}; /* not strictly inside (0, 5) */
  EXPECT(mla_oracle_decode_split(q, kc, table, seqlens, B, S_Q, H_Q, H_KV, D, DV, PAGE, PAGES, MAXB,
                                 0, 0.2, 0, bad_ptr, bad_cut, out2, lse2) != 0);

  /* scheduler: empty sequences, more parts than units, one part */
  const int32_t lens[6] = {0, 31, 0, 33, 1000, 0};
  for (int parts = 1; parts <= 64; parts *= 4) {
    int32_t *meta = malloc(sizeof(int32_t) * 8 * parts);
    int32_t splits[7];
    if (!meta) return 2;
    EXPECT(mla_oracle_schedule(lens, 6, 32, parts, 2, meta, splits) == 0);
    EXPECT(splits[0] == 0 && splits[6] >= 6);
    free(meta);
  }
  int32_t meta1[8], splits1[7];
  EXPECT(mla_oracle_schedule(lens, 6, 32, 0, 2, meta1, splits1) != 0);
  EXPECT(mla_oracle_schedule(lens, 6, 32, 1, 0, meta1, splits1) != 0);
  const int32_t neg[2] = {5, -1};
  EXPECT(mla_oracle_schedule(neg, 2, 32, 1, 1, meta1, splits1) != 0);

  free(q);
  free(kc);
  free(out);
  free(lse);
  free(out2);
  free(lse2);
  printf("oracle sanitizer harness: %d failures\n", failures);
  return failures ? 1 : 0;
}
