/*
 * PIVOT query-group indexer -- CPU oracle (declarations).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library under top_token_selection_pivot_amd/.
 *
 * What it computes follows the arXiv abstract page of "PIVOT: Efficient
 * Query-Group Indexing for Token-Level Sparse Attention" (English abstract):
 * group nearby queries, average each group into one proxy query, run one
 * shared full-prefix indexer scan per group to get a candidate set, then either
 * share the proxy top-k across the group (PIVOT-Reuse) or re-score the candidate
 * set with each member's own query and take an individual top-k (PIVOT-Refine).
 * The per-query scan, the top-k of positions and the causal prefix follow the
 * ai-systems-engineering.com tutorial "Sparse Attention의 Indexer", section
 * "선택용 Query와 Key로 위치 고르기" (Figure 1) and section "생성이 진행되면
 * 선택도 달라집니다".  The multi-head score
 *     S(q, w, s) = sum_h w[h] * max(0, q[h] . k_s)
 * (one key per token, shared by every head) is the reading adopted for the
 * tutorial's remark that real indexers use several indexer heads.
 *
 * Numeric model: inputs are the exact reals their codes denote; dot products
 * and scores are accumulated in double (d ascending inside a head, then h
 * ascending).  The proxy construction is part of the algorithm and is done in
 * binary32 exactly as documented in pivot_oracle.c, so that a binary32 GPU
 * implementation can match its codes bit for bit.
 */
#ifndef PIVOT_ORACLE_H
#define PIVOT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_BF16 = 0, ORC_FP8_E4M3 = 1 };
enum { ORC_DENSE = 0, ORC_REUSE = 1, ORC_REFINE = 2 };

/* A view of the indexer inputs.  q holds R query rows [R][H][D] of codes
 * (uint16 bf16 codes or uint8 OCP E4M3FN codes), q_scale [R] per-row scales
 * (fp8 only, NULL for bf16), w [R][H] head weights.  k holds N keys [N][D] of
 * codes, k_scale [N] per-key scales (fp8 only). */
typedef struct {
  int H, D, dtype;
  const void* q;
  const float* q_scale;
  const float* w;
  const void* k;
  const float* k_scale;
} orc_view;

/* Fills the oracle's constant tables; call once before using the oracle from
 * several host threads (each call is single-threaded and shares only these). */
void orc_init(void);

/* number formats */
double orc_bf16_value(uint16_t code);
double orc_e4m3_value(uint8_t code);
uint16_t orc_bf16_from_f32(float x);      /* round to nearest, ties to even */
uint8_t orc_e4m3_from_f32(float x);       /* nearest, ties to even, saturate to +-448 */

/* Score of a query (codes qc [H][D], scale qs, weights w [H]) against key s. */
double orc_score(const orc_view* v, const void* qc, float qs, const float* w, int s);

/* Exact top-m of an index pool: order by (score descending, position ascending),
 * keep the first min(m, n), emit them in ascending position order, pad with -1. */
void orc_topk(int n, const int32_t* pos, const double* score, int m, int32_t* out);

/* Proxy of the n consecutive query rows row0..row0+n-1.  Writes the proxy codes
 * [H][D] (same code type as the view), its scale (1 for bf16) and weights [H]. */
void orc_proxy(const orc_view* v, int row0, int n, void* codes_out, float* scale_out,
               float* w_out);

/* Dense indexer for the listed query rows (row t sits at position t and sees
 * keys [0, t]).  out: [nrows][topk]. */
void orc_dense_rows(const orc_view* v, const int32_t* rows, int nrows, int topk,
                    int32_t* out);

/* One query group: members are query rows row0..row0+n-1 sitting at positions
 * pos0..pos0+n-1; the proxy scan covers keys [0, pos0+n-1].
 * out: [n][topk].  cand_out (optional): [m] proxy top-m, m = C for REFINE,
 * topk for REUSE, unused for DENSE.  proxy_scores_out (optional): [pos0+n]. */
void orc_group(const orc_view* v, int row0, int pos0, int n, int topk, int C, int mode,
               int32_t* out, int32_t* cand_out, double* proxy_scores_out);

/* Prefill groups: the sequence has L queries and L keys, groups of g
 * consecutive queries aligned at position 0 (the last one may be partial).
 * For each listed group j writes out rows [j*g, e_j] into out_rows (packed in
 * the listed order, each group taking n_j rows) and, optionally, its
 * candidate list into cand_out[j_listed][m]. */
void orc_prefill_groups(const orc_view* v, int L, int g, int topk, int C, int mode,
                        const int32_t* groups, int ngroups, int32_t* out_rows,
                        int32_t* cand_out);

/* Variants with the sliding window excluded from the candidates: every query
 * at position t chooses among positions 0..t-excl only, and a group's proxy
 * scan covers 0..e-excl (e = its last member's position).  excl = 0 gives the
 * functions above. */
void orc_dense_rows_ex(const orc_view* v, const int32_t* rows, int nrows, int topk, int excl,
                       int32_t* out);
void orc_group_ex(const orc_view* v, int row0, int pos0, int n, int topk, int C, int mode,
                  int excl, int32_t* out, int32_t* cand_out, double* proxy_scores_out);
void orc_prefill_groups_ex(const orc_view* v, int L, int g, int topk, int C, int mode, int excl,
                           const int32_t* groups, int ngroups, int32_t* out_rows,
                           int32_t* cand_out);

/* Union of a selection sel [k] (ascending, -1 padded) with the sliding window
 * of size W at position t (positions max(0, t-W+1)..t): ascending, each
 * position once, -1 padded to k + W entries. */
void orc_window_union(const int32_t* sel, int k, int t, int W, int32_t* out);

/* Sparse main attention over the selected positions (multi-query layout,
 * computed in double): out[r][h] = sum over the valid selected s of
 * softmax_s(scale * q[r][h] . k_s) v_s.  q [R][Hq][d], k [.][d], v [.][dv] are
 * bf16 codes; row r reads sequence r / rows_per_seq, whose rows start at
 * (r / rows_per_seq) * seq_stride; idx [R][nidx] entries outside [0, seq_len)
 * are skipped; a row with none gets zeros.  out [R][Hq][dv]. */
void orc_sparse_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          const int32_t* idx, int R, int Hq, int d, int dv, int nidx,
                          int rows_per_seq, long seq_stride, int seq_len, double scale,
                          double* out);

/* Scores of the query row `row` of the view against keys [0, n). */
void orc_score_row(const orc_view* v, int row, int n, double* out);

/* Scores of the query row `row` against the n listed keys. */
void orc_score_list(const orc_view* v, int row, const int32_t* keys, int n, double* out);

/* Scores of arbitrary (query row, key) pairs. */
void orc_score_pairs(const orc_view* v, const int32_t* rows, const int32_t* keys, int npairs,
                     double* out);

#ifdef __cplusplus
}
#endif
#endif
