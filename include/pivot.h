/*
 * pivot.h -- C ABI of the PIVOT query-group indexer for MI355X (gfx950).
 *
 * The indexer of token-level sparse attention picks, for each query, the
 * positions of the top-k earlier tokens under an indexer score; the
 * tutorial "Sparse Attention의 Indexer" (ai-systems-engineering.com, Figure 1
 * and the section on how the selection changes during generation) shows the
 * plain version: score every key up to and including the query's own
 * position, keep the k best positions.  PIVOT ("PIVOT: Efficient Query-Group
 * Indexing for Token-Level Sparse Attention", arXiv:2607.24593, English
 * abstract on the arxivdaily page) replaces the per-query scan: a group of
 * nearby queries is averaged into one proxy query, the proxy scans the full
 * causal prefix once and keeps a candidate set, and then either every member
 * receives the proxy's top-k (PIVOT-Reuse) or every member re-scores the
 * candidates with its own query and keeps its own top-k (PIVOT-Refine).
 * Prefill groups are fixed-size runs of consecutive queries; in decode the
 * group is the set of queries one multi-token-prediction step produces.
 *
 * Score of query q (H heads of dimension D, head weights w) against key k_s
 * (one key per token, shared by all heads):
 *     S(q, s) = sum_h w[h] * max(0, q[h] . k_s)
 * with, for fp8, the positive per-token scales applied as s_q * s_k * S(codes).
 *
 * Conventions for every entry point below:
 *  - Tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates or frees device memory.  Scratch memory comes from the
 *    caller's `workspace` (256-byte aligned), sized by the *_workspace_size
 *    functions; a larger workspace lets the library process more score rows
 *    per pass, a smaller one (down to the size for one row block) is accepted.
 *  - Inputs are read-only; `out` and `workspace` must not alias any input.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and the call returns without synchronising.  Calls sharing a workspace
 *    must be ordered on one stream.
 *  - Arguments are validated on the host before anything is enqueued; on a
 *    non-zero status nothing was launched and `out` is untouched.  A failed
 *    launch returns PIVOT_ERR_HIP.  pivot_last_error_detail() gives a message
 *    for the last failure on the calling thread.
 *  - Codes: bf16 (uint16 storage) or OCP FP8 E4M3FN (uint8 storage, finite
 *    max 448) with one float32 scale per token, which must be > 0.  NaN or Inf
 *    inputs are outside the contract.
 *  - Supported shapes: 1 <= H <= 64; D in {32, 64, 128, 256} for bf16 and
 *    {64, 128, 256} for fp8; one sequence's keys (L*D or Lmax*D codes) below
 *    2 GiB.  q and k 16-byte aligned, w / scales / out
 *    4-byte aligned.
 *  - Output rows list positions in ascending order; a row holding fewer than
 *    topk positions is padded with -1 at its tail.  Among equal scores the
 *    lower position is preferred, so every output is unique.
 */
#ifndef PIVOT_H
#define PIVOT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PIVOT_OK = 0,
  PIVOT_ERR_NULL = 1,        /* a required pointer is NULL */
  PIVOT_ERR_SHAPE = 2,       /* L, B, H, Lmax, R ... out of range (e.g. L < 1, arrays too large) */
  PIVOT_ERR_PARAM = 3,       /* g, topk, C, mode, dtype, window ... invalid (e.g. C < topk for Refine) */
  PIVOT_ERR_UNSUPPORTED = 4, /* a valid shape the kernels are not built for (H > 64, D not in the set) */
  PIVOT_ERR_ALIGN = 5,       /* a pointer is not aligned as required */
  PIVOT_ERR_WORKSPACE = 6,   /* workspace smaller than the minimum */
  PIVOT_ERR_HIP = 7,         /* a kernel launch failed */
  PIVOT_ERR_INTERNAL = 8     /* an internal inconsistency (a bug in the library) */
} pivot_status_t;

typedef enum {
  PIVOT_MODE_DENSE = 0,  /* every query scans its own prefix (g is ignored) */
  PIVOT_MODE_REUSE = 1,  /* PIVOT-Reuse: members share the proxy top-k */
  PIVOT_MODE_REFINE = 2  /* PIVOT-Refine: members re-score the proxy top-C */
} pivot_mode_t;

typedef enum { PIVOT_BF16 = 0, PIVOT_FP8_E4M3 = 1 } pivot_dtype_t;

typedef enum {
  PIVOT_WINDOW_SHARED = 0,   /* the window's positions remain candidates; union with the selection */
  PIVOT_WINDOW_EXCLUDED = 1  /* the window is excluded from the candidates; topk chosen before it */
} pivot_window_mode_t;

int pivot_version(void);
const char* pivot_status_string(int status);
/* Message for the last failure on the calling thread (thread-local; "" if none). */
const char* pivot_last_error_detail(void);

/* ---------------------------------------------------------------------------
 * Prefill: one sequence of L queries over its own L keys (query t sits at
 * position t and sees keys 0..t).  Groups of g consecutive queries start at
 * position 0; the last group holds the remaining L mod g queries when g does
 * not divide L.  The proxy of group j (members j*g..e_j) scans keys 0..e_j.
 *
 *   q       [L][H][D] codes           q_scale [L] float (fp8 only, else NULL)
 *   w       [L][H] float head weights
 *   k       [L][D] codes              k_scale [L] float (fp8 only, else NULL)
 *   out     [L][topk] int32 positions
 *   out_scores  optional [L][topk] float (NULL: not written): the binary32
 *           score of each selected position as the kernels computed it (fp8:
 *           with s_q * s_k applied) -- the member's own score for DENSE and
 *           REFINE, the proxy's score for REUSE (the score that selected it);
 *           NaN where out holds -1.  For tolerance checks against a reference.
 *   C       candidate-set size for Refine (C >= topk); ignored otherwise
 * Returns a pivot_status_t.
 * ------------------------------------------------------------------------- */
size_t pivot_workspace_size(int L, int H, int D, int g, int topk, int C, int mode, int dtype);
size_t pivot_workspace_min_size(int L, int H, int D, int g, int topk, int C, int mode, int dtype);
int pivot_indexer(const void* q, const float* q_scale, const float* w, const void* k,
                  const float* k_scale, int L, int H, int D, int g, int topk, int C, int mode,
                  int dtype, int32_t* out, float* out_scores, void* workspace, size_t workspace_bytes,
                  void* stream);

/* ---------------------------------------------------------------------------
 * Decode: one multi-token-prediction step for B sequences.  Sequence b holds
 * cache_len[b] keys (the g new ones included) and decodes g queries at
 * positions cache_len[b]-g .. cache_len[b]-1; they form one group whose proxy
 * scans the whole cache 0..cache_len[b]-1.
 *
 *   q         [B][g][H][D] codes      q_scale [B][g] float (fp8 only)
 *   w         [B][g][H] float
 *   k_cache   [B][Lmax][D] codes      k_scale [B][Lmax] float (fp8 only)
 *   cache_len [B] int32, DEVICE memory; precondition g <= cache_len[b] <= Lmax
 *             (a sequence breaking it receives rows of -1)
 *   out       [B][g][topk] int32 positions
 *   out_scores optional [B][g][topk] float, as for pivot_indexer (NULL: not written)
 * ------------------------------------------------------------------------- */
size_t pivot_decode_workspace_size(int B, int Lmax, int H, int D, int g, int topk, int C,
                                   int mode, int dtype);
int pivot_indexer_decode(const void* q, const float* q_scale, const float* w,
                         const void* k_cache, const float* k_scale, const int32_t* cache_len,
                         int B, int Lmax, int H, int D, int g, int topk, int C, int mode,
                         int dtype, int32_t* out, float* out_scores, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Allocation-free decode step, for callers that cannot allocate device
 * memory around the call (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments and result as
 * pivot_indexer_decode, without a workspace: the scratch memory is a device
 * array inside this library, pivot_noalloc_scratch_bytes() bytes (128 MiB)
 * on every GPU the library runs on, held until the process ends.  A step
 * whose pivot_decode_workspace_size exceeds it returns PIVOT_ERR_WORKSPACE
 * (the decode workload of 32 sequences of up to 131072 fp8 keys with g = 2
 * fits in every mode).  The call uses the current device's copy (the stream
 * must belong to the current device); it allocates and frees nothing, and
 * every call clears what has to start at zero.  All calls on one GPU share
 * that GPU's array, so calls that overlap on one GPU (different streams or
 * threads without ordering) race: order them on one stream.
 * ------------------------------------------------------------------------- */
int pivot_indexer_decode_noalloc(const void* q, const float* q_scale, const float* w,
                                 const void* k_cache, const float* k_scale, const int32_t* cache_len,
                                 int B, int Lmax, int H, int D, int g, int topk, int C, int mode,
                                 int dtype, int32_t* out, float* out_scores, void* stream);
size_t pivot_noalloc_scratch_bytes(void);

/* ---------------------------------------------------------------------------
 * Prefill and decode with a sliding window added to every query's selection
 * (tutorial "Sparse Attention의 Indexer", section on combining the recent
 * window with the selected positions, Figure 3).  The window of size `window`
 * at position t holds the positions max(0, t-window+1) .. t; each query reads
 * the union of its window and its selection, each position once.
 *
 *   window_mode PIVOT_WINDOW_SHARED: the selection is the one pivot_indexer /
 *     pivot_indexer_decode make (the window's positions stay candidates), so
 *     a row holds up to topk + window positions and fewer when they overlap.
 *   window_mode PIVOT_WINDOW_EXCLUDED: the window is excluded from the
 *     candidates, so a query at t chooses its topk among 0..t-window; for a
 *     group the proxy's scan covers 0..e-window (e = its last member) and
 *     every member keeps the candidates <= its own t-window.  A row holds
 *     min(topk, max(0, t-window+1)) + min(window, t+1) positions.
 *
 * Arguments as for pivot_indexer / pivot_indexer_decode, plus window >= 0
 * and window_mode; out is [L][topk + window] (prefill) or
 * [B][g][topk + window] (decode), ascending, -1 padded.  The workspace sizes
 * are those of the calls without a window.  window = 0 with either mode gives
 * the rows of the calls without a window.
 * ------------------------------------------------------------------------- */
int pivot_indexer_window(const void* q, const float* q_scale, const float* w, const void* k,
                         const float* k_scale, int L, int H, int D, int g, int topk, int C,
                         int mode, int dtype, int window, int window_mode, int32_t* out,
                         void* workspace, size_t workspace_bytes, void* stream);
int pivot_indexer_decode_window(const void* q, const float* q_scale, const float* w,
                                const void* k_cache, const float* k_scale, const int32_t* cache_len,
                                int B, int Lmax, int H, int D, int g, int topk, int C, int mode,
                                int dtype, int window, int window_mode, int32_t* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * One decode step (as pivot_indexer_decode_window) over a paged indexer-key
 * cache, as a server keeps it: the keys of every sequence live in pages of a
 * shared pool, and a block table lists each sequence's pages in order.  The
 * result is the one pivot_indexer_decode_window gives for the contiguous cache
 * whose position p of sequence b holds the pool row
 *     block_table[b][p / page_size] * page_size + p % page_size.
 *
 *   k_pages        [num_pages][page_size][D] codes (16-byte aligned)
 *   k_scale_pages  [num_pages][page_size] float (fp8 only, else NULL)
 *   block_table    [B][max_pages] int32, DEVICE memory: the first
 *                  ceil(cache_len[b] / page_size) entries of row b are page
 *                  ids; an id outside [0, num_pages) reads as a page of zero
 *                  keys (scores 0), never out of bounds
 *   page_size      a power of two, 64 .. 2^20 (every 64-key tile pair of the
 *                  scan lies in one page)
 *   cache_len      [B] int32, DEVICE memory; g <= cache_len[b] <=
 *                  max_pages * page_size, else the sequence's rows are -1
 * The pool must stay below 4 GiB of key codes.  The workspace is
 * pivot_decode_workspace_size(B, max_pages * page_size, ...) bytes.  Other
 * arguments as for pivot_indexer_decode_window (window = 0: none).
 * ------------------------------------------------------------------------- */
int pivot_indexer_decode_paged(const void* q, const float* q_scale, const float* w, const void* k_pages,
                               const float* k_scale_pages, int num_pages, int page_size,
                               const int32_t* block_table, int max_pages, const int32_t* cache_len, int B,
                               int H, int D, int g, int topk, int C, int mode, int dtype, int window,
                               int window_mode, int32_t* out, void* workspace, size_t workspace_bytes,
                               void* stream);

/* ---------------------------------------------------------------------------
 * Several prefill sequences of different lengths in one call.  Sequence i
 * holds rows cu_seqlens[i] .. cu_seqlens[i+1]-1 of q, w, k (and the scales):
 * its queries see only its own keys (position t of the sequence sees its keys
 * 0..t), and its groups start at its first row.  Every sequence's rows are
 * exactly those pivot_indexer_window would give for that sequence alone.
 *
 *   cu_seqlens  [nseq + 1] int64, HOST memory, cu_seqlens[0] = 0, non-decreasing
 *               (a zero-length sequence is allowed)
 *   out         [cu_seqlens[nseq]][topk + window] int32
 *   window, window_mode as for pivot_indexer_window (window = 0: none)
 * All sequences are validated before anything is enqueued.  They then run
 * concurrently on up to four streams the library owns (created once per
 * device, default priority), forked from `stream` and joined back to it with
 * events, each stream with its own slice of the workspace: the call is
 * ordered on `stream` like any other.  pivot_varlen_workspace_size gives room
 * for one slice per stream (the longest sequence's preferred size each); a
 * smaller workspace runs fewer sequences at a time, down to one after
 * another on `stream` (it must hold at least the longest sequence's minimum).
 * ------------------------------------------------------------------------- */
size_t pivot_varlen_workspace_size(const int64_t* cu_seqlens, int nseq, int H, int D, int g, int topk,
                                   int C, int mode, int dtype);
int pivot_indexer_varlen(const void* q, const float* q_scale, const float* w, const void* k,
                         const float* k_scale, const int64_t* cu_seqlens, int nseq, int H, int D, int g,
                         int topk, int C, int mode, int dtype, int window, int window_mode, int32_t* out,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Cross-layer index reuse stacked on the indexer (molayo1419.me "PIVOT
 * explained", section Try it now and the Sources list: IndexCache,
 * "Accelerating Sparse Attention via Cross-Layer Index Reuse", stacked on
 * PIVOT; only the title is on the pages).  A model has nlayers layers, each
 * with its own indexer inputs.  A layer with full[l] != 0 runs the indexer
 * (as pivot_indexer / pivot_indexer_decode, in the given mode); every other
 * layer reuses the index rows of the nearest full layer before it, so layer
 * 0 must be full.  Reusing layers skip their indexer entirely; their rows
 * are copied from the source layer unless the caller passes the same out
 * pointer for both (then nothing is written for the reusing layer).
 *
 *   full        [nlayers] int32, HOST memory
 *   q, q_scale, w, k (k_cache), k_scale, out
 *               HOST arrays of nlayers DEVICE pointers, each laid out as for
 *               pivot_indexer (prefill) or pivot_indexer_decode (decode);
 *               entries of reusing layers other than out are not read
 *               (q_scale / k_scale arrays may be NULL for bf16)
 *   cache_len   decode: one [B] array shared by every layer (device)
 * Every full layer is validated before anything is enqueued; the layers then
 * run in order on `stream`, sharing one workspace of pivot_workspace_size
 * (pivot_decode_workspace_size) bytes.
 * ------------------------------------------------------------------------- */
int pivot_indexer_layers(int nlayers, const int32_t* full, const void* const* q, const float* const* q_scale,
                         const float* const* w, const void* const* k, const float* const* k_scale, int L, int H,
                         int D, int g, int topk, int C, int mode, int dtype, int32_t* const* out, void* workspace,
                         size_t workspace_bytes, void* stream);
int pivot_indexer_decode_layers(int nlayers, const int32_t* full, const void* const* q, const float* const* q_scale,
                                const float* const* w, const void* const* k_cache, const float* const* k_scale,
                                const int32_t* cache_len, int B, int Lmax, int H, int D, int g, int topk, int C,
                                int mode, int dtype, int32_t* const* out, void* workspace, size_t workspace_bytes,
                                void* stream);

/* ---------------------------------------------------------------------------
 * Sparse main attention over the selected positions (tutorial "Sparse
 * Attention의 Indexer", text after Figure 1): the main query of a row scores
 * the main keys at the positions the indexer selected and combines the values
 * there with softmax weights over those positions only:
 *     out[r][h] = sum_s softmax_s(scale * q[r][h] . k_s) v_s,  s in idx[r].
 * Multi-query layout: one key row and one value row per position, shared by
 * the Hq query heads.  bf16 codes; d = dv = 128; Hq in {32, 64}.
 *
 *   q    [R][Hq][d]       out [R][Hq][dv] float (16-byte aligned)
 *   k    key rows of d codes, v value rows of dv codes: row r reads sequence
 *        r / rows_per_seq, whose rows start at row (r / rows_per_seq) *
 *        seq_stride (one sequence: rows_per_seq = R, seq_stride unused)
 *   idx  [R][nidx] int32 positions in the row's sequence (an indexer output,
 *        e.g. pivot_indexer's rows); entries outside [0, seq_len) are skipped
 *        and a row with none gets zeros
 *   scale  > 0, applied to every dot product (usually 1/sqrt(d))
 * One sequence's key rows (and its value rows) must stay below 2 GiB
 * (PIVOT_ERR_SHAPE).  Scores and sums are binary32; the softmax weights enter the value product
 * as two bf16 terms, so the result is close to binary32 accuracy.  Few rows
 * split their slots over several waves and need a workspace of
 * pivot_sparse_attention_workspace_size bytes (0: none needed).
 * ------------------------------------------------------------------------- */
size_t pivot_sparse_attention_workspace_size(int R, int Hq, int dv, int nidx);
int pivot_sparse_attention(const void* q, const void* k, const void* v, const int32_t* idx, int R,
                           int Hq, int d, int dv, int nidx, int rows_per_seq, long long seq_stride,
                           int seq_len, float scale, float* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Single steps of the prefill path, for step-level checks.
 *
 * pivot_proxy_mean: the proxy of every group (arXiv:2607.24593 abstract: one
 * proxy query stands for the whole group; molayo1419.me "PIVOT explained",
 * section How It Works: the proxy is the mean of the group).  Members are added
 * in ascending position in binary32 and divided by the member count; w is
 * averaged the same way.  bf16: the mean is rounded to nearest even.  fp8: a
 * fresh scale s = amax/448 (1 if all zero) and codes rounded to nearest even,
 * saturating at +-448.  A one-member group is copied unchanged.  Also serves
 * decode rows laid out [B][g][...] by passing L = B*g.
 *   qbar [G][H][D] codes, qbar_scale [G] float (written for both dtypes,
 *   1 for bf16), wbar [G][H] float, G = ceil(L/g).
 *
 * pivot_candidates: proxy mean, the proxy's full-prefix scan and its top-m
 * (m = C for REFINE, topk for REUSE): cand [G][m] ascending, -1 padded.
 *
 * pivot_decode_candidates: the same three steps for a decode step (one group
 * per sequence, the scan covering its whole cache): cand [B][m].
 *
 * pivot_dbg_score_rows: the indexer score rows themselves (tutorial "Sparse
 * Attention의 Indexer", Figure 1: each query scores every key of its causal
 * prefix), as the full-prefix scan kernel computes them.  Query row r of
 * q [R][H][D] (with w [R][H], q_scale [R] for fp8) sees keys 0..p(r),
 * p(r) = min(r * pos_mul + pos_add, Lk - 1), of k [Lk][D] (k_scale [Lk]):
 *     S[(r - row_begin) * ldS + s] = sum_h w[r][h] * max(0, q[r][h] . k[s])
 * (times q_scale[r] * k_scale[s] for fp8) for row_begin <= r < row_end and
 * s <= p(r); every other entry of S is left untouched.  Dense rows are
 * pos_mul = 1, pos_add = 0; the proxies of pivot_proxy_mean are rows of
 * qbar with pos_mul = g, pos_add = g - 1.  ldS >= p(row_end - 1) + 1.
 * ------------------------------------------------------------------------- */
int pivot_proxy_mean(const void* q, const float* q_scale, const float* w, int L, int H, int D,
                     int g, int dtype, void* qbar, float* qbar_scale, float* wbar, void* stream);
int pivot_candidates(const void* q, const float* q_scale, const float* w, const void* k,
                     const float* k_scale, int L, int H, int D, int g, int topk, int C, int mode,
                     int dtype, int32_t* cand, void* workspace, size_t workspace_bytes,
                     void* stream);
int pivot_decode_candidates(const void* q, const float* q_scale, const float* w,
                            const void* k_cache, const float* k_scale, const int32_t* cache_len,
                            int B, int Lmax, int H, int D, int g, int topk, int C, int mode,
                            int dtype, int32_t* cand, void* workspace, size_t workspace_bytes,
                            void* stream);
int pivot_dbg_score_rows(const void* q, const float* q_scale, const float* w, const void* k,
                         const float* k_scale, int R, int Lk, int H, int D, int dtype, int row_begin,
                         int row_end, int pos_mul, int pos_add, float* S, long long ldS, void* stream);

/* ---------------------------------------------------------------------------
 * Per-kernel timing for measurement tools.  While enabled (process-wide),
 * every kernel the library launches is bracketed by two HIP events recorded on
 * its launch stream.  pivot_profile_read waits for the recorded events, writes
 * the summed milliseconds and the launch count of each kernel class
 * (PIVOT_K_* order; arrays of n entries) and clears the record.  Disabled by
 * default.  Returns a pivot_status_t.
 * ------------------------------------------------------------------------- */
enum {
  PIVOT_K_PROXY = 0,        /* proxy mean */
  PIVOT_K_SCAN = 1,         /* prefill full-prefix scan (proxies or dense queries) */
  PIVOT_K_SELECT = 2,       /* proxy top-m / dense top-k */
  PIVOT_K_REFINE = 3,       /* Refine gather-score */
  PIVOT_K_MEMBER_SELECT = 4,/* Refine member top-k */
  PIVOT_K_BROADCAST = 5,    /* Reuse broadcast */
  PIVOT_K_DECODE_SCAN = 6,  /* decode key-cache scan */
  PIVOT_K_WINDOW = 7,       /* sliding-window union */
  PIVOT_K_ATTENTION = 8,    /* sparse main attention (and its chunk merge) */
  PIVOT_K_LAYER_COPY = 9,   /* index rows handed to a reusing layer */
  PIVOT_K_COUNT = 10
};
int pivot_profile_enable(int on);
int pivot_profile_read(double* ms, long long* launches, int n);

/* ---------------------------------------------------------------------------
 * Layout self-test of the matrix-core instructions the scoring kernels use
 * (32x32 bf16 and fp8 tiles): writes, for each lane l and accumulator i,
 * the row, the column and a k-pairing probe into out[3][2][64][16] (device,
 * int32): [0] rows, [1] columns, [2] pairing (1 where the lane halves' k
 * slices pair up as the kernels assume), for bf16 then fp8.
 * ------------------------------------------------------------------------- */
int pivot_selftest_mfma_layout(int32_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PIVOT_H */
