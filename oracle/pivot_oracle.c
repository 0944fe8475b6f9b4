/*
 * PIVOT query-group indexer -- CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.  Plain,
 * single-threaded, slow on purpose; every function states the passage it
 * follows.  Pages cited:
 *   [ABS]  arxivdaily page for arXiv:2607.24593, "PIVOT: Efficient Query-Group
 *          Indexing for Token-Level Sparse Attention", English abstract.
 *   [BLOG] molayo1419.me, "PIVOT explained: from paper to working code",
 *          section "How It Works" (pseudocode: the proxy is the group mean).
 *   [TUT]  ai-systems-engineering.com, "Sparse Attention의 Indexer", Figure 1
 *          (score by dot product, top-3 of positions) and the section on how
 *          the selection changes during generation (causal prefix, self
 *          included).
 * Readings taken where the pages are silent are listed in pivot_oracle.h and
 * next to the code that takes them.
 */
#include "pivot_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats.                                                           */
/* ------------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32 word. */
double orc_bf16_value(uint16_t code) {
  uint32_t bits = (uint32_t)code << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* OCP 8-bit E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent field 0 is subnormal (m/8 * 2^-6); exponent 15 with mantissa 7 is
 * NaN; there is no infinity; the largest finite magnitude is 448. */
double orc_e4m3_value(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* binary32 -> bf16, round to nearest, ties to even: pick the nearer of the two
 * bf16 neighbours (the one that truncates toward zero and the next one up in
 * magnitude); on a tie the one whose code is even. */
uint16_t orc_bf16_from_f32(float x) {
  uint32_t bits;
  memcpy(&bits, &x, sizeof bits);
  if (isnan(x)) return (uint16_t)((bits >> 16) | 0x0040u);
  uint16_t lo = (uint16_t)(bits >> 16);
  uint16_t hi = (uint16_t)(lo + 1u);
  double ax = fabs((double)x);
  double vlo = fabs(orc_bf16_value(lo));
  double vhi = fabs(orc_bf16_value(hi)); /* may be +inf past the largest finite */
  double dlo = ax - vlo, dhi = vhi - ax;
  if (dlo < dhi) return lo;
  if (dhi < dlo) return hi;
  return (lo & 1u) ? hi : lo;
}

/* binary32 -> E4M3FN, round to nearest, ties to even, saturating to +-448:
 * the positive codes 0x00..0x7E are increasing in value, so binary-search the
 * nearest neighbours in that table and pick the nearer one (even code on a
 * tie). */
uint8_t orc_e4m3_from_f32(float x) {
  if (isnan(x)) return 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  int lo = 0, hi = 0x7E; /* invariant: value(lo) <= a < value(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (orc_e4m3_value((uint8_t)mid) <= a)
      lo = mid;
    else
      hi = mid;
  }
  double dlo = a - orc_e4m3_value((uint8_t)lo);
  double dhi = orc_e4m3_value((uint8_t)hi) - a;
  int pick;
  if (dlo < dhi)
    pick = lo;
  else if (dhi < dlo)
    pick = hi;
  else
    pick = (lo & 1) ? hi : lo;
  return (uint8_t)(sign | pick);
}

/* ------------------------------------------------------------------------ */
/* Score ([TUT] Figure 1 for one head; several weighted ReLU heads as read). */
/* ------------------------------------------------------------------------ */

static double e4m3_table[256];
static int e4m3_table_ready = 0;

static double code_value(int dtype, const void* base, long idx) {
  if (dtype == ORC_BF16) return orc_bf16_value(((const uint16_t*)base)[idx]);
  if (!e4m3_table_ready) {
    for (int c = 0; c < 256; ++c) e4m3_table[c] = orc_e4m3_value((uint8_t)c);
    e4m3_table_ready = 1;
  }
  return e4m3_table[((const uint8_t*)base)[idx]];
}

static const void* code_ptr(int dtype, const void* base, long idx) {
  if (dtype == ORC_BF16) return (const uint16_t*)base + idx;
  return (const uint8_t*)base + idx;
}

/* The n values denoted by the codes starting at base[idx]. */
static void decode_codes(int dtype, const void* base, long idx, int n, double* out) {
  for (int i = 0; i < n; ++i) out[i] = code_value(dtype, base, idx + i);
}

/* S = sum_h w[h] * max(0, sum_d q[h][d] * k_s[d]) on decoded values qd [H][D]
 * and kd [D]; d ascending inside a head, then h ascending. */
static double score_decoded(int H, int D, const double* qd, const float* w, const double* kd) {
  double total = 0.0;
  for (int h = 0; h < H; ++h) {
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += qd[(long)h * D + d] * kd[d];
    double relu = dot > 0.0 ? dot : 0.0;
    total += (double)w[h] * relu;
  }
  return total;
}

/* Score of the decoded query qd (scale qs, weights w) against key s.  For fp8
 * the values are scale * e4m3(code); the positive per-token scales are taken
 * out of the sums (ReLU and the sums are positively homogeneous), which keeps
 * the code dot product exact in double: every code product is a multiple of
 * 2^-18 below 2^18, and D of them fit in 53 bits. */
static double score_key(const orc_view* v, const double* qd, float qs, const float* w, int s,
                        double* kd) {
  decode_codes(v->dtype, v->k, (long)s * v->D, v->D, kd);
  double total = score_decoded(v->H, v->D, qd, w, kd);
  if (v->dtype == ORC_FP8_E4M3) total = total * (double)qs * (double)v->k_scale[s];
  return total;
}

/* Scores of one query (codes qc) against the listed keys (keys 0..n-1 when
 * keys is NULL). */
static void score_keys(const orc_view* v, const void* qc, float qs, const float* w,
                       const int32_t* keys, int n, double* out) {
  double* qd = (double*)malloc(sizeof(double) * (size_t)v->H * v->D);
  double* kd = (double*)malloc(sizeof(double) * (size_t)v->D);
  decode_codes(v->dtype, qc, 0, v->H * v->D, qd);
  for (int i = 0; i < n; ++i) out[i] = score_key(v, qd, qs, w, keys ? keys[i] : i, kd);
  free(qd);
  free(kd);
}

double orc_score(const orc_view* v, const void* qc, float qs, const float* w, int s) {
  double r;
  int32_t key = s;
  score_keys(v, qc, qs, w, &key, 1, &r);
  return r;
}

static float row_scale(const orc_view* v, int row) {
  return v->dtype == ORC_FP8_E4M3 ? v->q_scale[row] : 1.0f;
}

void orc_score_row(const orc_view* v, int row, int n, double* out) {
  const void* qc = code_ptr(v->dtype, v->q, (long)row * v->H * v->D);
  score_keys(v, qc, row_scale(v, row), v->w + (long)row * v->H, NULL, n, out);
}

void orc_score_pairs(const orc_view* v, const int32_t* rows, const int32_t* keys, int npairs,
                     double* out) {
  for (int i = 0; i < npairs; ++i) {
    const void* qc = code_ptr(v->dtype, v->q, (long)rows[i] * v->H * v->D);
    score_keys(v, qc, row_scale(v, rows[i]), v->w + (long)rows[i] * v->H, keys + i, 1, out + i);
  }
}

/* ------------------------------------------------------------------------ */
/* Top-m ([TUT] Figure 1: keep the positions of the m largest scores).       */
/* Reading: equal scores go to the lower position; the result is listed in   */
/* ascending position order and padded with -1.                              */
/* ------------------------------------------------------------------------ */

typedef struct {
  double score;
  int32_t pos;
} scored_pos;

static int by_score_desc_pos_asc(const void* pa, const void* pb) {
  const scored_pos* a = (const scored_pos*)pa;
  const scored_pos* b = (const scored_pos*)pb;
  if (a->score > b->score) return -1; /* -0.0 and +0.0 compare equal here */
  if (a->score < b->score) return 1;
  return (a->pos > b->pos) - (a->pos < b->pos);
}

static int by_int_asc(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

void orc_topk(int n, const int32_t* pos, const double* score, int m, int32_t* out) {
  scored_pos* tmp = (scored_pos*)malloc(sizeof(scored_pos) * (size_t)(n > 0 ? n : 1));
  for (int i = 0; i < n; ++i) {
    tmp[i].score = score[i];
    tmp[i].pos = pos[i];
  }
  qsort(tmp, (size_t)n, sizeof(scored_pos), by_score_desc_pos_asc);
  int keep = n < m ? n : m;
  for (int i = 0; i < keep; ++i) out[i] = tmp[i].pos;
  qsort(out, (size_t)keep, sizeof(int32_t), by_int_asc);
  for (int i = keep; i < m; ++i) out[i] = -1;
  free(tmp);
}

/* ------------------------------------------------------------------------ */
/* Proxy query ([BLOG] the proxy is the group mean; [ABS] one proxy query    */
/* stands for the group).  Readings: the head weights are averaged the same  */
/* way; the mean is taken in binary32, adding the members in ascending       */
/* position and dividing by the member count; the result is rounded back to */
/* the input type (bf16 round-to-nearest-even, or for fp8 a fresh per-proxy  */
/* scale amax/448 and round-to-nearest-even saturating codes).  A group of   */
/* one member is that member, codes, scale and weights unchanged.            */
/* ------------------------------------------------------------------------ */

void orc_proxy(const orc_view* v, int row0, int n, void* codes_out, float* scale_out,
               float* w_out) {
  const int H = v->H, D = v->D, HD = H * D;
  if (n == 1) {
    size_t esz = v->dtype == ORC_BF16 ? 2 : 1;
    memcpy(codes_out, code_ptr(v->dtype, v->q, (long)row0 * HD), esz * (size_t)HD);
    *scale_out = row_scale(v, row0);
    memcpy(w_out, v->w + (long)row0 * H, sizeof(float) * (size_t)H);
    return;
  }
  float* mean = (float*)malloc(sizeof(float) * (size_t)HD);
  for (int e = 0; e < HD; ++e) {
    float sum = 0.0f;
    for (int t = row0; t < row0 + n; ++t) {
      float x = (float)code_value(v->dtype, v->q, (long)t * HD + e);
      if (v->dtype == ORC_FP8_E4M3) x = v->q_scale[t] * x; /* one binary32 product */
      sum = sum + x;
    }
    mean[e] = sum / (float)n;
  }
  for (int h = 0; h < H; ++h) {
    float sum = 0.0f;
    for (int t = row0; t < row0 + n; ++t) sum = sum + v->w[(long)t * H + h];
    w_out[h] = sum / (float)n;
  }
  if (v->dtype == ORC_BF16) {
    for (int e = 0; e < HD; ++e) ((uint16_t*)codes_out)[e] = orc_bf16_from_f32(mean[e]);
    *scale_out = 1.0f;
  } else {
    float amax = 0.0f;
    for (int e = 0; e < HD; ++e) {
      float a = fabsf(mean[e]);
      if (a > amax) amax = a;
    }
    float sp = amax > 0.0f ? amax / 448.0f : 1.0f;
    for (int e = 0; e < HD; ++e) ((uint8_t*)codes_out)[e] = orc_e4m3_from_f32(mean[e] / sp);
    *scale_out = sp;
  }
  free(mean);
}

/* ------------------------------------------------------------------------ */
/* Dense indexer ([TUT] Figure 1 and the generation section: query t scores */
/* every key 0..t, itself included, and keeps the top-k positions).          */
/* ------------------------------------------------------------------------ */

void orc_dense_rows(const orc_view* v, const int32_t* rows, int nrows, int topk,
                    int32_t* out) {
  orc_dense_rows_ex(v, rows, nrows, topk, 0, out);
}

/* Window excluded from the candidates ([TUT] section "최근 window와 선택한
 * 위치 결합하기", the alternative design): query t chooses among keys
 * 0..t-excl only (none when t < excl). */
void orc_dense_rows_ex(const orc_view* v, const int32_t* rows, int nrows, int topk, int excl,
                       int32_t* out) {
  for (int i = 0; i < nrows; ++i) {
    int t = rows[i] - excl;
    int n = t + 1 > 0 ? t + 1 : 0;
    double* sc = (double*)malloc(sizeof(double) * (size_t)n);
    int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    orc_score_row(v, rows[i], n, sc);
    for (int s = 0; s < n; ++s) pos[s] = s;
    orc_topk(n, pos, sc, topk, out + (long)i * topk);
    free(sc);
    free(pos);
  }
}

/* ------------------------------------------------------------------------ */
/* One group ([ABS]): proxy -> one shared full-prefix scan -> candidate set  */
/* -> Reuse (share the proxy top-k) or Refine (each member re-scores the     */
/* candidates with its own query and weights and keeps its own top-k).       */
/* Readings: the shared scan covers keys up to and including the last        */
/* member's position; member t never receives a position after t.           */
/* ------------------------------------------------------------------------ */

void orc_group(const orc_view* v, int row0, int pos0, int n, int topk, int C, int mode,
               int32_t* out, int32_t* cand_out, double* proxy_scores_out) {
  orc_group_ex(v, row0, pos0, n, topk, C, mode, 0, out, cand_out, proxy_scores_out);
}

/* The same with the window excluded from the candidates ([TUT] section
 * "최근 window와 선택한 위치 결합하기", the alternative design).  Reading for
 * a group: member t chooses among positions 0..t-excl, so the proxy's scan,
 * which serves every member, covers 0..e-excl (the last member's range). */
void orc_group_ex(const orc_view* v, int row0, int pos0, int n, int topk, int C, int mode,
                  int excl, int32_t* out, int32_t* cand_out, double* proxy_scores_out) {
  const int H = v->H, D = v->D;
  const int e = pos0 + n - 1 - excl; /* last position any member may choose */
  const int nk = e + 1 > 0 ? e + 1 : 0; /* keys 0..e */

  if (mode == ORC_DENSE) {
    for (int i = 0; i < n; ++i) {
      int t = pos0 + i - excl;
      int nt = t + 1 > 0 ? t + 1 : 0;
      double* sc = (double*)malloc(sizeof(double) * (size_t)(nt + 1));
      int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nt + 1));
      const void* qc = code_ptr(v->dtype, v->q, (long)(row0 + i) * H * D);
      score_keys(v, qc, row_scale(v, row0 + i), v->w + (long)(row0 + i) * H, NULL, nt, sc);
      for (int s = 0; s < nt; ++s) pos[s] = s;
      orc_topk(nt, pos, sc, topk, out + (long)i * topk);
      free(sc);
      free(pos);
    }
    return;
  }

  size_t esz = v->dtype == ORC_BF16 ? 2 : 1;
  void* pq = malloc(esz * (size_t)H * D);
  float ps;
  float* pw = (float*)malloc(sizeof(float) * (size_t)H);
  orc_proxy(v, row0, n, pq, &ps, pw);

  double* psc = (double*)malloc(sizeof(double) * (size_t)(nk + 1));
  int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nk + 1));
  score_keys(v, pq, ps, pw, NULL, nk, psc);
  for (int s = 0; s < nk; ++s) pos[s] = s;
  if (proxy_scores_out) memcpy(proxy_scores_out, psc, sizeof(double) * (size_t)nk);

  if (mode == ORC_REUSE) {
    int32_t* ptop = (int32_t*)malloc(sizeof(int32_t) * (size_t)topk);
    orc_topk(nk, pos, psc, topk, ptop);
    if (cand_out) memcpy(cand_out, ptop, sizeof(int32_t) * (size_t)topk);
    for (int i = 0; i < n; ++i) {
      int t = pos0 + i - excl;
      int32_t* o = out + (long)i * topk;
      int c = 0;
      for (int j = 0; j < topk; ++j)
        if (ptop[j] >= 0 && ptop[j] <= t) o[c++] = ptop[j];
      for (; c < topk; ++c) o[c] = -1;
    }
    free(ptop);
  } else { /* ORC_REFINE */
    int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)C);
    orc_topk(nk, pos, psc, C, cand);
    if (cand_out) memcpy(cand_out, cand, sizeof(int32_t) * (size_t)C);
    double* msc = (double*)malloc(sizeof(double) * (size_t)C);
    int32_t* mpos = (int32_t*)malloc(sizeof(int32_t) * (size_t)C);
    for (int i = 0; i < n; ++i) {
      int t = pos0 + i - excl;
      const void* qc = code_ptr(v->dtype, v->q, (long)(row0 + i) * H * D);
      int np = 0;
      for (int j = 0; j < C; ++j)
        if (cand[j] >= 0 && cand[j] <= t) mpos[np++] = cand[j];
      score_keys(v, qc, row_scale(v, row0 + i), v->w + (long)(row0 + i) * H, mpos, np, msc);
      orc_topk(np, mpos, msc, topk, out + (long)i * topk);
    }
    free(cand);
    free(msc);
    free(mpos);
  }
  free(psc);
  free(pos);
  free(pq);
  free(pw);
}

/* Prefill grouping ([ABS]: fixed-size groups of consecutive queries in
 * prefill).  Reading: groups are aligned at position 0 and the last one holds
 * the remaining L mod g queries when g does not divide L. */
void orc_prefill_groups(const orc_view* v, int L, int g, int topk, int C, int mode,
                        const int32_t* groups, int ngroups, int32_t* out_rows,
                        int32_t* cand_out) {
  orc_prefill_groups_ex(v, L, g, topk, C, mode, 0, groups, ngroups, out_rows, cand_out);
}

void orc_prefill_groups_ex(const orc_view* v, int L, int g, int topk, int C, int mode, int excl,
                           const int32_t* groups, int ngroups, int32_t* out_rows,
                           int32_t* cand_out) {
  int m = mode == ORC_REFINE ? C : topk;
  long row = 0;
  for (int i = 0; i < ngroups; ++i) {
    int j = groups[i];
    int first = j * g;
    int n = (first + g <= L) ? g : L - first;
    orc_group_ex(v, first, first, n, topk, C, mode, excl, out_rows + row * topk,
                 cand_out ? cand_out + (long)i * m : NULL, NULL);
    row += n;
  }
}

/* ------------------------------------------------------------------------ */
/* Sliding window added to a selection ([TUT] section "최근 window와 선택한  */
/* 위치 결합하기", Figure 3): the window of size W at position t holds the   */
/* positions max(0, t-W+1) .. t; the positions read are the union of the     */
/* window and the selection, each position once.  Output: ascending,        */
/* padded with -1 to k + W entries.                                          */
/* ------------------------------------------------------------------------ */

void orc_window_union(const int32_t* sel, int k, int t, int W, int32_t* out) {
  int32_t* all = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k + W + 1));
  int n = 0;
  for (int i = 0; i < k; ++i)
    if (sel[i] >= 0) all[n++] = sel[i];
  for (int s = t - W + 1; s <= t; ++s)
    if (s >= 0) all[n++] = s;
  qsort(all, (size_t)n, sizeof(int32_t), by_int_asc);
  int c = 0;
  for (int i = 0; i < n; ++i)
    if (c == 0 || all[i] != out[c - 1]) out[c++] = all[i];
  for (; c < k + W; ++c) out[c] = -1;
  free(all);
}

/* ------------------------------------------------------------------------ */
/* Sparse main attention over the selected positions ([TUT] text after      */
/* Figure 1: the main query scores the main keys at the selected positions  */
/* only, and the values there are combined with softmax weights over those  */
/* positions; the indexer scores are not the weights).  Reading: standard   */
/* scaled dot-product attention, one key and one value row per position     */
/* shared by all query heads (multi-query layout).  Computed in double.     */
/* q [R][Hq][d] bf16 codes; k [nseq][seq_stride][d], v [nseq][seq_stride][dv] */
/* bf16 codes; row r belongs to sequence r / rows_per_seq; idx [R][nidx]    */
/* positions, entries outside [0, seq_len) are skipped; out [R][Hq][dv].    */
/* A row with no selected position gets zeros.                              */
/* ------------------------------------------------------------------------ */

void orc_sparse_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          const int32_t* idx, int R, int Hq, int d, int dv, int nidx,
                          int rows_per_seq, long seq_stride, int seq_len, double scale,
                          double* out) {
  double* sc = (double*)malloc(sizeof(double) * (size_t)(nidx > 0 ? nidx : 1));
  for (int r = 0; r < R; ++r) {
    const long base = (long)(r / rows_per_seq) * seq_stride;
    const int32_t* sel = idx + (long)r * nidx;
    for (int h = 0; h < Hq; ++h) {
      double* o = out + ((long)r * Hq + h) * dv;
      for (int c = 0; c < dv; ++c) o[c] = 0.0;
      const uint16_t* qh = q + ((long)r * Hq + h) * d;
      double mx = -INFINITY;
      for (int i = 0; i < nidx; ++i) {
        sc[i] = -INFINITY;
        if (sel[i] < 0 || sel[i] >= seq_len) continue;
        const uint16_t* kr = k + (base + sel[i]) * d;
        double dot = 0.0;
        for (int e = 0; e < d; ++e) dot += orc_bf16_value(qh[e]) * orc_bf16_value(kr[e]);
        sc[i] = dot * scale;
        if (sc[i] > mx) mx = sc[i];
      }
      if (mx == -INFINITY) continue; /* nothing selected */
      double den = 0.0;
      for (int i = 0; i < nidx; ++i) {
        if (sc[i] == -INFINITY) continue;
        double p = exp(sc[i] - mx);
        den += p;
        const uint16_t* vr = v + (base + sel[i]) * dv;
        for (int c = 0; c < dv; ++c) o[c] += p * orc_bf16_value(vr[c]);
      }
      for (int c = 0; c < dv; ++c) o[c] /= den;
    }
  }
  free(sc);
}

/* Fills the E4M3 value table up front, so that later calls only read it
 * (calls from several host threads then share no writes). */
void orc_init(void) {
  for (int c = 0; c < 256; ++c) e4m3_table[c] = orc_e4m3_value((uint8_t)c);
  e4m3_table_ready = 1;
}

/* Scores of the query row `row` of the view against the listed keys (the same
 * score as orc_score_row, for an arbitrary key list). */
void orc_score_list(const orc_view* v, int row, const int32_t* keys, int n, double* out) {
  const void* qc = code_ptr(v->dtype, v->q, (long)row * v->H * v->D);
  score_keys(v, qc, row_scale(v, row), v->w + (long)row * v->H, keys, n, out);
}
