// pivot_kernels.h -- argument blocks and launch wrappers of the PIVOT kernels
// (internal to libpivot; the public ABI is include/pivot.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pivot {

// Proxy mean over groups of g consecutive rows of q[R][H][D].  Optionally
// also clears nzero words at `zero` (a later kernel's counters).
struct ProxyArgs {
  const uint8_t* q;
  const float* q_scale;
  const float* w;
  int R, H, D, g;
  uint8_t* qbar;
  float* qbar_scale;
  float* wbar;
  uint32_t* zero = nullptr;
  size_t nzero = 0;
};

// Causal scan of query rows [row_begin, row_end) against keys k[0..Lk).
// Row r sees keys 0..pos(r), pos(r) = min(r*pos_mul + pos_add, pos_cap), and
// writes its scores to S + (r - row_begin)*ldS.
struct ScanArgs {
  const uint8_t* q;
  const float* q_scale;
  const float* w;
  const uint8_t* k;
  const float* k_scale;
  int Lk, H;
  int row_begin, row_end;
  int pos_mul, pos_add, pos_cap;
  int kc;  // keys per workgroup (multiple of 32)
  float* S;
  long long ldS;
  int nchunks = 0, nblocks = 0;  // key chunks and row blocks (set by the launcher)
};

// Members of groups [grp_begin, grp_end) score their group's candidates.
// kind 0 (prefill): group j = rows [j*g, min(L, j*g+g)), keys k[0..L).
// kind 1 (decode):  group j = rows [j*g, j*g+g) of sequence j, keys
//                   k[j*Lmax ...], cache_len[j] keys.
// Candidates of group j: cand + (j - grp_begin)*ldc, m slots, ascending, -1 tail.
// Member row r writes slot scores to S + (r - row_base)*ldS.
struct RefineArgs {
  const uint8_t* q;
  const float* q_scale;
  const float* w;
  const uint8_t* k;
  const float* k_scale;
  int H, kind, L, g, Lmax;
  const int32_t* cache_len;
  int grp_begin, grp_end;
  const int32_t* cand;
  int ldc, m;
  int slot_chunk;
  float* S;
  long long ldS;
  int row_base;
  int excl = 0;  // window excluded: every member's limit is its position - excl
  // Decode with a paged key cache (bt non-NULL): position p of sequence j is
  // row bt[j * bt_stride + (p >> page_shift)] * 2^page_shift + p % 2^page_shift
  // of the pool k (k_scale), which holds pool_rows rows (below 4 GiB of keys);
  // a page id outside [0, pool_rows >> page_shift) reads as zero keys.
  const int32_t* bt = nullptr;
  int bt_stride = 0, page_shift = 0;
  int pool_rows = 0;
};

// Decode scan: for each sequence b, qr query rows (rows b*qr .. b*qr+qr-1 of
// q) scan the sequence's cache_len[b] keys.  qr == 1: the proxy, which sees
// every key; otherwise the g members, member i seeing keys 0..n_b-g+i.
// Persistent workgroups take equal runs of work over the batch's pairs of
// 32-key tiles (a sequence's pairs plus kDecSegmentPairs units for a segment's
// set-up); `hist` (optional, zeroed beforehand) receives for every output row
// the histogram of the top 12 bits of its scores' order-preserving keys,
// [B*qr][4096].
struct DecScanArgs {
  const uint8_t* q;
  const float* q_scale;
  const float* w;
  const uint8_t* k;
  const float* k_scale;
  int Lmax, H;
  const int32_t* cache_len;
  int g, qr;
  float* S;
  long long ldS;
  uint32_t* hist;
  int B;
  int excl = 0;  // window excluded: every row's limit moves down by excl
  // paged key cache (bt non-NULL), addressed as in RefineArgs; pages hold a
  // multiple of 64 keys so that every pair of 32-key tiles lies in one page
  const int32_t* bt = nullptr;
  int bt_stride = 0, page_shift = 0;
  int num_pages = 0;
};

constexpr int kSelectCapDefault = 7680;  // keys a long-row selection stages in LDS

// Top-m of decode score rows with precomputed first-digit histograms: `parts`
// workgroups per row gather the keys at or above the threshold bin of their
// slice into per-slice regions ([nrows][parts][kTopkCap] keys and slots,
// counts [nrows][parts], -1 if the threshold bin is too crowded), the first
// of them also storing the row's threshold bin and the count of keys above it
// in `thr` ([nrows][2]), then one workgroup per row finishes the selection.
struct DecSelectArgs {
  const float* S;
  long long ldS;
  int nrows, m;
  int kind;  // kLenCache or kLenDecodeDense
  int g, Lmax;
  const int32_t* cache_len;
  const uint32_t* hist;
  int parts;
  uint32_t* ckey;
  int32_t* cslot;
  int32_t* ccount;
  int32_t* out;
  long long ldo;
  int excl = 0;  // window excluded: row lengths shrink by excl
  uint32_t* thr = nullptr;  // per row: first-digit threshold bin, keys in higher bins
  float* out_s = nullptr;   // optional: score of every output entry (NaN for -1), stride ldos
  long long ldos = 0;
  int cap = kSelectCapDefault;  // keys each slice region of ckey / cslot holds
};

// Row-length rules of the top-m selection.
enum : int {
  kLenPos = 0,         // n = pos(R) + 1, positions = slots
  kLenCache = 1,       // decode proxy row b: n = cache_len[b]
  kLenDecodeDense = 2, // decode member row b*g+i: n = cache_len[b] - g + i + 1
  kLenRefine = 3,      // member row: n = #candidates <= its position, positions = cand[slot]
};

struct TopkArgs {
  const float* S;
  long long ldS;
  int row_begin, nrows;
  int m;
  int32_t* out;
  long long ldo;
  int kind;
  int pos_mul, pos_add, pos_cap;  // kLenPos
  int decode;                     // kLenRefine: 0 prefill, 1 decode
  int g, Lmax;
  const int32_t* cache_len;
  const int32_t* map;  // kLenRefine: candidate lists
  int ldmap, map_grp_begin;
  int excl = 0;        // kLenRefine / kLenCache / kLenDecodeDense: limits move down by excl
  float* out_s = nullptr;  // optional: score of every output entry (NaN for -1), stride ldos
  long long ldos = 0;
};

// Reuse: member rows [row_begin, row_end) receive their group's proxy top-k
// clipped to their own prefix.
struct BroadcastArgs {
  const int32_t* ptop;
  int ldp, grp_begin;
  int32_t* out;
  int topk;
  int decode, g, Lmax;
  const int32_t* cache_len;
  int row_begin, row_end;
  long long ldo = 0;  // output row stride (0: topk)
  int excl = 0;       // window excluded: member t keeps entries <= t - excl
  // optional scores: out_s[i][s] = the proxy's score S[j - grp_begin][position]
  // (NaN for -1); S holds the proxy score rows of groups grp_begin.. (stride ldS)
  const float* S = nullptr;
  long long ldS = 0;
  float* out_s = nullptr;
  long long ldos = 0;
};

// Sliding window added in place to selected rows: row i of out (stride ldo)
// holds its selection in the first topk entries (ascending, -1 padded); the
// row becomes the selection's entries below the window, then the window
// max(0, t-W+1)..t, then -1 up to topk + W entries.  Row i's position t:
// prefill row_begin + i; decode cache_len[b] - g + i % g for row i = b*g + i%g
// (rows of an invalid sequence stay -1).
struct WindowArgs {
  int32_t* out;
  long long ldo;
  int rows, topk, W;
  int decode, g, Lmax;
  const int32_t* cache_len;
  int row_begin;
};

// Sparse main attention (multi-query, bf16 codes, D = DV = 128, Hq in {32, 64}):
// row r reads sequence r / rows_per_seq, whose key and value rows start at row
// (r / rows_per_seq) * seq_stride of k and v; idx [R][nidx] entries outside
// [0, seq_len) are skipped.  Each of the nch chunks of a row covers `chunk`
// slots (a multiple of 32); with nch == 1 the output [R][Hq][DV] is written
// directly, otherwise part_o [R][nch][Hq][DV] and part_ml [R][nch][2][Hq]
// (running maximum, then sum) are merged by a second kernel.
struct SAttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  int R, Hq, nidx;
  int rows_per_seq;
  long long seq_stride;
  int seq_len;
  float scale;
  int chunk, nch;
  float* out;
  float* part_o;
  float* part_ml;
};

hipError_t launch_proxy_mean(const ProxyArgs& a, int dtype, hipStream_t st);
hipError_t launch_scan(const ScanArgs& a, int dtype, int D, hipStream_t st);
hipError_t launch_refine(const RefineArgs& a, int dtype, int D, hipStream_t st);
hipError_t launch_decode_scan(const DecScanArgs& a, int dtype, int D, hipStream_t st);
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);
hipError_t launch_broadcast(const BroadcastArgs& a, hipStream_t st);
hipError_t launch_selftest_mfma(int32_t* out, hipStream_t st);
hipError_t launch_decode_select(const DecSelectArgs& a, hipStream_t st);
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t st);
hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, size_t n, hipStream_t st);
hipError_t launch_window_union(const WindowArgs& a, hipStream_t st);

#ifndef PIVOT_DEC_SEGMENT_PAIRS
#define PIVOT_DEC_SEGMENT_PAIRS 32
#endif
constexpr int kDecSegmentPairs = PIVOT_DEC_SEGMENT_PAIRS;  // a decode segment's set-up, in pairs of work
constexpr int kRefineSlotLimit = 4096;  // candidate slots one Refine workgroup holds
constexpr int kSelectCap = kSelectCapDefault;
constexpr int kSelectBins1 = 4096;   // bins of the first radix digit (top 12 bits)

bool score_shape_supported(int dtype, int D);
bool sattn_shape_supported(int Hq, int d, int dv);
hipError_t launch_sparse_attention(const SAttnArgs& a, hipStream_t st);

}  // namespace pivot
