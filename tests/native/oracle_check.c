/*
 * The fp64 oracle (oracle/mla_oracle.c) built with AddressSanitizer and
 * UndefinedBehaviorSanitizer and driven over its edge cases on tiny inputs:
 * every input dtype, dense and sparse lists, split mode, row subsets, empty
 * sequences, queries that see nothing, padded and out-of-range indices, a
 * page id out of range and invalid arguments.  Exit status 0 when every call
 * returned what it should; a sanitizer report exits non-zero.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int mla_oracle_decode(const void* q_nope, const void* q_pe, int q_dtype, double q_scale, const void* kv,
                      int kv_dtype, double kv_scale, const int32_t* block_table, const int32_t* seq_lens,
                      const int32_t* topk_indices, int K, int B, int T, int H, int NB, int P, int MB,
                      double softmax_scale, int num_splits, const int64_t* rows, int64_t n_rows, double* out,
                      double* lse, int n_threads);

enum { BF16 = 0, E4M3 = 1, F64 = 2 };

static int failures = 0;
#define CHECK(c, msg)                                       \
  do {                                                      \
    if (!(c)) {                                             \
      fprintf(stderr, "check failed: %s (%s)\n", #c, msg); \
      failures++;                                           \
    }                                                       \
  } while (0)

static uint32_t rng_state = 12345u;
static uint32_t next_u32(void) {
  rng_state = rng_state * 1664525u + 1013904223u;
  return rng_state;
}
static double uniform(void) { return (next_u32() >> 8) / 16777216.0 * 2.0 - 1.0; }

enum { B = 3, T = 2, H = 4, P = 16, MB = 4, NB = 10, K = 7 };

int main(void) {
  const int64_t nq = (int64_t)B * T * H;
  double* qn = malloc(sizeof(double) * nq * 512);
  double* qp = malloc(sizeof(double) * nq * 64);
  double* kv = malloc(sizeof(double) * NB * P * 576);
  uint16_t* qn16 = malloc(2 * nq * 512);
  uint16_t* qp16 = malloc(2 * nq * 64);
  uint16_t* kv16 = malloc(2 * NB * P * 576);
  uint8_t* qn8 = malloc(nq * 512);
  uint8_t* qp8 = malloc(nq * 64);
  uint8_t* kv8 = malloc(NB * P * 576);
  double* out = malloc(sizeof(double) * nq * 512);
  double* lse = malloc(sizeof(double) * nq);
  for (int64_t i = 0; i < nq * 512; i++) qn[i] = uniform();
  for (int64_t i = 0; i < nq * 64; i++) qp[i] = uniform();
  for (int64_t i = 0; i < NB * P * 576; i++) kv[i] = uniform();
  /* bf16 / e4m3 bytes: arbitrary patterns, NaN codes included (only where no list reaches) */
  for (int64_t i = 0; i < nq * 512; i++) { qn16[i] = (uint16_t)(0x3c00 + (next_u32() & 0x3ff)); qn8[i] = (uint8_t)(next_u32() & 0x77); }
  for (int64_t i = 0; i < nq * 64; i++) { qp16[i] = (uint16_t)(0x3c00 + (next_u32() & 0x3ff)); qp8[i] = (uint8_t)(next_u32() & 0x77); }
  for (int64_t i = 0; i < NB * P * 576; i++) { kv16[i] = (uint16_t)(0xbc00 + (next_u32() & 0x3ff)); kv8[i] = (uint8_t)(next_u32() & 0xf6); }

  /* sequence 0: empty; 1: one token; 2: 50 tokens over 4 pages */
  const int32_t lens[B] = {0, 1, 50};
  const int32_t bt[B * MB] = {-1, -1, -1, -1, 7, -1, -1, -1, 3, 0, 9, 5};
  int32_t idx[B * T * K];
  for (int i = 0; i < B * T * K; i++) idx[i] = (int32_t)(next_u32() % 70) - 10;   /* -10 .. 59: some out of range */

  const double scale = 0.0721687836;
  const void* qs[3][2] = {{qn16, qp16}, {qn8, qp8}, {qn, qp}};
  const void* kvs[3] = {kv16, kv8, kv};
  for (int dt = 0; dt < 3; dt++) {
    for (int sp = 0; sp < 2; sp++) {
      for (int splits = 0; splits < 4; splits++) {
        int st = mla_oracle_decode(qs[dt][0], qs[dt][1], dt, 0.5, kvs[dt], dt, 0.25, bt, lens, sp ? idx : NULL, K, B,
                                   T, H, NB, P, MB, scale, splits, NULL, 0, out, lse, 1);
        CHECK(st == 0, "decode");
        for (int64_t r = 0; r < nq; r++) {
          const int b = (int)(r / (T * H));
          if (b == 0) CHECK(isinf(lse[r]) && lse[r] < 0 && out[r * 512] == 0.0, "empty sequence");
          else if (!sp) CHECK(isfinite(lse[r]) || (b == 1 && (r / H) % T == 0), "finite lse");
          for (int d = 0; d < 512; d++) CHECK(isfinite(out[r * 512 + d]), "finite out");
        }
      }
    }
  }
  /* one visible token: out is that token's latent (f64 input) */
  {
    int st = mla_oracle_decode(qn, qp, F64, 1.0, kv, F64, 1.0, bt, lens, NULL, 0, B, T, H, NB, P, MB, scale, 0, NULL,
                               0, out, lse, 1);
    CHECK(st == 0, "decode f64");
    const int64_t r = (int64_t)(1 * T + 1) * H + 2;   /* b=1, t=1: sees token 0 */
    for (int d = 0; d < 512; d++) CHECK(out[r * 512 + d] == kv[(7 * P + 0) * 576 + d], "kv_len=1 closed form");
  }
  /* row subset, in any order */
  {
    const int64_t rows[3] = {nq - 1, 0, 9};
    int st = mla_oracle_decode(qn, qp, F64, 1.0, kv, F64, 1.0, bt, lens, NULL, 0, B, T, H, NB, P, MB, scale, 2, rows,
                               3, out, lse, 1);
    CHECK(st == 0, "rows");
    const int64_t bad_rows[1] = {nq};
    st = mla_oracle_decode(qn, qp, F64, 1.0, kv, F64, 1.0, bt, lens, NULL, 0, B, T, H, NB, P, MB, scale, 0, bad_rows,
                           1, out, lse, 1);
    CHECK(st == -1, "row out of range");
  }
  /* a page id out of range, a table too short for the length */
  {
    int32_t bt_bad[B * MB] = {-1, -1, -1, -1, 7, -1, -1, -1, 3, 0, NB, 5};
    int st = mla_oracle_decode(qn, qp, F64, 1.0, kv, F64, 1.0, bt_bad, lens, NULL, 0, B, T, H, NB, P, MB, scale, 0,
                               NULL, 0, out, lse, 1);
    CHECK(st == -2, "page out of range");
    const int32_t long_lens[B] = {0, 1, 65};
    st = mla_oracle_decode(qn, qp, F64, 1.0, kv, F64, 1.0, bt, long_lens, NULL, 0, B, T, H, NB, P, MB, scale, 0,
                           NULL, 0, out, lse, 1);
    CHECK(st == -2, "length beyond the table");
  }
  /* invalid arguments */
  CHECK(mla_oracle_decode(qn, qp, 7, 1.0, kv, F64, 1.0, bt, lens, NULL, 0, B, T, H, NB, P, MB, scale, 0, NULL, 0, out,
                          lse, 1) == -1, "dtype");
  CHECK(mla_oracle_decode(qn, qp, F64, 1.0, kv, F64, 1.0, bt, lens, NULL, 0, B, 0, H, NB, P, MB, scale, 0, NULL, 0,
                          out, lse, 1) == -1, "T=0");
  CHECK(mla_oracle_decode(qn, qp, F64, 1.0, kv, F64, 1.0, bt, lens, idx, -1, B, T, H, NB, P, MB, scale, 0, NULL, 0,
                          out, lse, 1) == -1, "K<0");
  CHECK(mla_oracle_decode(qn, qp, F64, 1.0, kv, F64, 1.0, bt, lens, NULL, 0, 0, T, H, NB, P, MB, scale, 0, NULL, 0,
                          out, lse, 1) == 0, "B=0");

  free(qn); free(qp); free(kv); free(qn16); free(qp16); free(kv16); free(qn8); free(qp8); free(kv8);
  free(out); free(lse);
  printf("oracle sanitizer check: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
