/*
 * Drives every entry of the CPU oracle (oracle/pivot_oracle.c) over many tiny
 * shapes so that a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * sees each loop, index and buffer of it: partial groups, g larger than L,
 * topk and C larger than the prefix, excluded windows, both code types, and
 * sparse attention rows with padding.  It also checks the structure every
 * selection must have (ascending positions, -1 only at the tail, causal).
 * Test infrastructure only: built and run by tests/test_oracle_sanitize.py.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pivot_oracle.h"

static unsigned long long rng_state = 0x9E3779B97F4A7C15ull;
static unsigned next_u32(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (unsigned)(rng_state >> 11);
}
static float small_value(void) { return (float)((int)(next_u32() % 9) - 4) / 8.0f; }

static int failures = 0;
static void check_row(const int32_t* row, int width, int limit, const char* what) {
  int last = -1, tail = 0;
  for (int i = 0; i < width; ++i) {
    const int v = row[i];
    if (v < 0) {
      tail = 1;
      if (v != -1) ++failures;
      continue;
    }
    if (tail || v <= last || v > limit) {
      fprintf(stderr, "bad %s row entry %d at %d (limit %d)\n", what, v, i, limit);
      ++failures;
    }
    last = v;
  }
}

static void run_shape(int dtype, int L, int H, int D, int g, int topk, int C, int excl) {
  const size_t esz = dtype == ORC_BF16 ? 2 : 1;
  void* q = malloc((size_t)L * H * D * esz);
  void* k = malloc((size_t)L * D * esz);
  float* w = malloc((size_t)L * H * sizeof(float));
  float* qs = dtype == ORC_BF16 ? NULL : malloc((size_t)L * sizeof(float));
  float* ks = dtype == ORC_BF16 ? NULL : malloc((size_t)L * sizeof(float));
  for (size_t i = 0; i < (size_t)L * H * D; ++i) {
    if (dtype == ORC_BF16) ((uint16_t*)q)[i] = orc_bf16_from_f32(small_value());
    else ((uint8_t*)q)[i] = orc_e4m3_from_f32(small_value() * 64.0f);
  }
  for (size_t i = 0; i < (size_t)L * D; ++i) {
    if (dtype == ORC_BF16) ((uint16_t*)k)[i] = orc_bf16_from_f32(small_value());
    else ((uint8_t*)k)[i] = orc_e4m3_from_f32(small_value() * 64.0f);
  }
  for (size_t i = 0; i < (size_t)L * H; ++i) w[i] = (float)(1 + next_u32() % 4) / 8.0f;
  for (int i = 0; qs && i < L; ++i) qs[i] = 0.25f + (float)(next_u32() % 4) / 8.0f;
  for (int i = 0; ks && i < L; ++i) ks[i] = 0.5f + (float)(next_u32() % 4) / 8.0f;
  orc_view v = {H, D, dtype, q, qs, w, k, ks};

  const int G = (L + g - 1) / g;
  int32_t* groups = malloc((size_t)G * sizeof(int32_t));
  for (int j = 0; j < G; ++j) groups[j] = j;
  int32_t* out = malloc((size_t)L * topk * sizeof(int32_t));
  const int m = C > topk ? C : topk;
  int32_t* cand = malloc((size_t)G * m * sizeof(int32_t));
  for (int mode = ORC_DENSE; mode <= ORC_REFINE; ++mode) {
    orc_prefill_groups_ex(&v, L, g, topk, C, mode, excl, groups, G, out, mode == ORC_DENSE ? NULL : cand);
    for (int t = 0; t < L; ++t) check_row(out + (size_t)t * topk, topk, t - excl, "prefill");
  }
  int32_t* rows = malloc((size_t)L * sizeof(int32_t));
  for (int t = 0; t < L; ++t) rows[t] = t;
  orc_dense_rows_ex(&v, rows, L, topk, excl, out);
  for (int t = 0; t < L; ++t) check_row(out + (size_t)t * topk, topk, t - excl, "dense");

  /* the window union on each dense row, and pairwise scores */
  const int W = 3;
  int32_t* un = malloc((size_t)(topk + W) * sizeof(int32_t));
  for (int t = 0; t < L; ++t) {
    orc_window_union(out + (size_t)t * topk, topk, t, W, un);
    check_row(un, topk + W, t, "window");
  }
  double* sc = malloc((size_t)L * sizeof(double));
  orc_score_row(&v, L - 1, L, sc);
  orc_score_pairs(&v, rows, rows, L, sc);

  /* one proxy of the last (possibly partial) group */
  void* pc = malloc((size_t)H * D * esz);
  float ps, pw[64];
  orc_proxy(&v, (G - 1) * g, L - (G - 1) * g, pc, &ps, pw);

  free(pc); free(sc); free(un); free(rows); free(cand); free(out); free(groups);
  free(ks); free(qs); free(w); free(k); free(q);
}

static void run_attention(int R, int Hq, int d, int nidx, int seq_len) {
  uint16_t* q = malloc((size_t)R * Hq * d * 2);
  uint16_t* k = malloc((size_t)seq_len * d * 2);
  uint16_t* vv = malloc((size_t)seq_len * d * 2);
  int32_t* idx = malloc((size_t)R * nidx * sizeof(int32_t));
  double* out = malloc((size_t)R * Hq * d * sizeof(double));
  for (size_t i = 0; i < (size_t)R * Hq * d; ++i) q[i] = orc_bf16_from_f32(small_value());
  for (size_t i = 0; i < (size_t)seq_len * d; ++i) k[i] = orc_bf16_from_f32(small_value());
  for (size_t i = 0; i < (size_t)seq_len * d; ++i) vv[i] = orc_bf16_from_f32(small_value());
  for (size_t i = 0; i < (size_t)R * nidx; ++i) {
    const int r = (int)(next_u32() % (unsigned)(seq_len + 3)) - 2;  /* some outside the sequence */
    idx[i] = r;
  }
  orc_sparse_attention(q, k, vv, idx, R, Hq, d, d, nidx, R, 0, seq_len, 0.125, out);
  free(out); free(idx); free(vv); free(k); free(q);
}

int main(void) {
  const int Ls[] = {1, 2, 5, 17, 40};
  const int gs[] = {1, 2, 3, 8, 64};
  const int ks[] = {1, 3, 8};
  for (int dt = ORC_BF16; dt <= ORC_FP8_E4M3; ++dt)
    for (int a = 0; a < 5; ++a)
      for (int b = 0; b < 5; ++b)
        for (int c = 0; c < 3; ++c)
          for (int excl = 0; excl <= 2; excl += 2) {
            const int topk = ks[c];
            run_shape(dt, Ls[a], 1 + (a + b) % 3, dt == ORC_BF16 ? 2 + 2 * (b % 2) : 4, gs[b], topk,
                      topk + (a % 3) * 4, excl);
          }
  for (int i = 0; i < 4; ++i) run_attention(1 + i, 2, 8, 5 + i, 3 + 4 * i);
  /* the codecs over every code and a spread of values */
  for (int c = 0; c < 256; ++c) (void)orc_e4m3_value((uint8_t)c);
  for (int c = 0; c < 65536; c += 7) (void)orc_bf16_value((uint16_t)c);
  for (int i = -2000; i <= 2000; ++i) {
    (void)orc_e4m3_from_f32((float)i * 0.37f);
    (void)orc_bf16_from_f32((float)i * 1e-3f);
  }
  if (failures) {
    fprintf(stderr, "%d structural failures\n", failures);
    return 1;
  }
  printf("oracle sanitizer driver: ok\n");
  return 0;
}
