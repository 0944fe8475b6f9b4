// pivot_api.hip -- C ABI of the PIVOT indexer (declared in include/pivot.h):
// argument validation, workspace planning and the sequence of kernel launches
// on the caller's stream.  No device memory is allocated here.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/pivot.h"
#include "pivot_kernels.h"

using namespace pivot;

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 64;  // devices whose per-device state the library tracks
constexpr int kScanRowsPerLaunch = 1024;          // scan rows per launch within a pass
constexpr size_t kScoreBudget = size_t(2) << 30;  // preferred score bytes per pass
constexpr int kScanKeyChunk = 2048;              // keys per scan workgroup
constexpr int kRefineSlotChunk = 1024;           // candidate slots per refine workgroup

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
long long round_up(long long x, long long m) { return (x + m - 1) / m * m; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int esize(int dtype) { return dtype == PIVOT_BF16 ? 2 : 1; }

// ---------------------------------------------------------------------------
// Prefill plan.  Rows are proxies (REUSE/REFINE, one per group) or queries
// (DENSE).  Score rows of one pass live in one region, reused by the Refine
// member scores of the same pass.
// ---------------------------------------------------------------------------
struct PrefillPlan {
  int G;           // groups (= L for DENSE)
  int m;           // proxy selection size: C (REFINE) or topk
  long long ldS;   // score row stride (floats)
  long long ldR;   // refine member row stride (floats)
  size_t off_qbar, off_qs, off_wbar, off_cand, off_S;
  size_t per_row;  // bytes of score region per row (group)
  size_t fixed;    // bytes before the chunked part
  size_t per_chunk_row;
};

PrefillPlan plan_prefill(int L, int H, int D, int g, int topk, int C, int mode, int dtype) {
  PrefillPlan p{};
  const bool dense = mode == PIVOT_MODE_DENSE;
  p.G = dense ? L : (L + g - 1) / g;
  p.m = mode == PIVOT_MODE_REFINE ? C : topk;
  p.ldS = round_up(L, 64);
  p.ldR = round_up(C, 64);
  size_t off = 0;
  if (!dense) {
    p.off_qbar = off;
    off = align_up(off + (size_t)p.G * H * D * esize(dtype));
    p.off_qs = off;
    off = align_up(off + (size_t)p.G * 4);
    p.off_wbar = off;
    off = align_up(off + (size_t)p.G * H * 4);
  }
  p.fixed = off;
  size_t srow = (size_t)p.ldS * 4;
  if (mode == PIVOT_MODE_REFINE) srow = std::max(srow, (size_t)g * (size_t)p.ldR * 4);
  p.per_row = srow;
  p.per_chunk_row = srow + (dense ? 0 : (size_t)p.m * 4);
  return p;
}

// Workspace bytes for `rows` rows per pass.
size_t prefill_bytes(const PrefillPlan& p, int rows, bool dense) {
  size_t cand = dense ? 0 : align_up((size_t)rows * p.m * 4);
  return p.fixed + cand + align_up((size_t)rows * p.per_row) + kAlign;
}

int chunk_rows_for(const PrefillPlan& p, size_t ws, bool dense) {
  // all rows, else the largest multiple of 8 rows that fits
  if (prefill_bytes(p, p.G, dense) <= ws) return p.G;
  if (ws <= p.fixed) return 0;
  long long rows = (long long)((ws - p.fixed) / p.per_chunk_row) / 8 * 8 + 8;
  rows = std::min<long long>(rows, (long long)p.G / 8 * 8);
  while (rows > 0 && prefill_bytes(p, (int)rows, dense) > ws) rows -= 8;
  return (int)rows;
}

int validate_common(const void* q, const float* q_scale, const float* w, const void* k,
                    const float* k_scale, int H, int D, int g, int topk, int C, int mode,
                    int dtype) {
  if (dtype != PIVOT_BF16 && dtype != PIVOT_FP8_E4M3)
    return fail(PIVOT_ERR_PARAM, "dtype %d is not PIVOT_BF16 or PIVOT_FP8_E4M3", dtype);
  if (mode != PIVOT_MODE_DENSE && mode != PIVOT_MODE_REUSE && mode != PIVOT_MODE_REFINE)
    return fail(PIVOT_ERR_PARAM, "mode %d is not DENSE, REUSE or REFINE", mode);
  if (!q || !w || !k) return fail(PIVOT_ERR_NULL, "q, w and k must be non-NULL");
  if (dtype == PIVOT_FP8_E4M3 && (!q_scale || !k_scale))
    return fail(PIVOT_ERR_NULL, "fp8 inputs need q_scale and k_scale");
  if (H < 1) return fail(PIVOT_ERR_SHAPE, "H=%d must be >= 1", H);
  if (H > 64) return fail(PIVOT_ERR_UNSUPPORTED, "H=%d: the kernels hold at most 64 heads", H);
  if (!score_shape_supported(dtype, D))
    return fail(PIVOT_ERR_UNSUPPORTED, "D=%d unsupported for %s", D, dtype == PIVOT_BF16 ? "bf16" : "fp8");
  if (g < 1) return fail(PIVOT_ERR_PARAM, "g=%d must be >= 1", g);
  if (topk < 1) return fail(PIVOT_ERR_PARAM, "topk=%d must be >= 1", topk);
  if (mode == PIVOT_MODE_REFINE && C < topk)
    return fail(PIVOT_ERR_PARAM, "Refine needs C >= topk (C=%d, topk=%d)", C, topk);
  if (!aligned(q, 16) || !aligned(k, 16)) return fail(PIVOT_ERR_ALIGN, "q and k must be 16-byte aligned");
  if (!aligned(w, 4) || (q_scale && !aligned(q_scale, 4)) || (k_scale && !aligned(k_scale, 4)))
    return fail(PIVOT_ERR_ALIGN, "w and scales must be 4-byte aligned");
  return PIVOT_OK;
}

int validate_window(int window, int wmode, int topk) {
  if (wmode != PIVOT_WINDOW_SHARED && wmode != PIVOT_WINDOW_EXCLUDED)
    return fail(PIVOT_ERR_PARAM, "window_mode %d is not SHARED or EXCLUDED", wmode);
  if (window < 0) return fail(PIVOT_ERR_PARAM, "window=%d must be >= 0", window);
  if ((long long)topk + window > (1ll << 30)) return fail(PIVOT_ERR_PARAM, "topk + window too large");
  return PIVOT_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PIVOT_OK;
  return fail(PIVOT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Optional per-launch event timing (pivot_profile_enable).
struct TimedLaunch {
  int cls;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
std::vector<TimedLaunch> g_prof;

struct ProfileScope {
  hipStream_t st;
  int cls;
  hipEvent_t a = nullptr, b = nullptr;
  ProfileScope(int cls_, hipStream_t st_) : st(st_), cls(cls_) {
    if (!g_prof_on.load(std::memory_order_relaxed)) return;
    if (hipEventCreate(&a) != hipSuccess) {
      a = nullptr;
      return;
    }
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      a = nullptr;
      return;
    }
    if (hipEventRecord(a, st) != hipSuccess) drop();
  }
  void drop() {
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    a = b = nullptr;
  }
  ~ProfileScope() {
    if (!a) return;
    if (hipEventRecord(b, st) != hipSuccess) {
      drop();
      return;
    }
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof.push_back({cls, a, b});
  }
};

#define PIVOT_LAUNCH_K(cls, st, expr, what)           \
  do {                                                \
    ProfileScope prof_(cls, st);                      \
    int st_ = hip_status((expr), what);               \
    if (st_ != PIVOT_OK) return st_;                  \
  } while (0)

#define PIVOT_LAUNCH(expr, what)                      \
  do {                                                \
    int st_ = hip_status((expr), what);               \
    if (st_ != PIVOT_OK) return st_;                  \
  } while (0)

// Runs the prefill path.  `cand_user` (optional) receives every group's top-m
// and skips the member step (pivot_candidates).
// `outs` (optional, no window) receives the score of every output entry.
int run_prefill(const void* q, const float* q_scale, const float* w, const void* k,
                const float* k_scale, int L, int H, int D, int g, int topk, int C, int mode,
                int dtype, int32_t* out, int32_t* cand_user, void* workspace,
                size_t workspace_bytes, void* stream, int window = 0, int wmode = 0,
                float* outs = nullptr) {
  int st = validate_common(q, q_scale, w, k, k_scale, H, D, g, topk, C, mode, dtype);
  if (st) return st;
  st = validate_window(window, wmode, topk);
  if (st) return st;
  // window excluded from the candidates: every limit moves down by the window
  const int excl = wmode == PIVOT_WINDOW_EXCLUDED ? window : 0;
  const long long ldo = (long long)topk + window;
  if (L < 1) return fail(PIVOT_ERR_SHAPE, "L=%d must be >= 1", L);
  if ((long long)L * H * D > (1ll << 40)) return fail(PIVOT_ERR_SHAPE, "L*H*D too large");
  if ((long long)L * D * esize(dtype) >= (1ll << 31))
    return fail(PIVOT_ERR_SHAPE, "the key array (L*D codes) must stay below 2 GiB");
  if (!out && !cand_user) return fail(PIVOT_ERR_NULL, "out must be non-NULL");
  if ((out && !aligned(out, 4)) || (cand_user && !aligned(cand_user, 4)) || (outs && !aligned(outs, 4)))
    return fail(PIVOT_ERR_ALIGN, "output must be 4-byte aligned");
  if (outs && window > 0) return fail(PIVOT_ERR_INTERNAL, "scores are written without a window only");
  if (!workspace) return fail(PIVOT_ERR_NULL, "workspace must be non-NULL");
  if (!aligned(workspace, kAlign)) return fail(PIVOT_ERR_ALIGN, "workspace must be 256-byte aligned");
  const bool dense = mode == PIVOT_MODE_DENSE;
  if (dense) g = 1;
  const PrefillPlan p = plan_prefill(L, H, D, g, topk, C, mode, dtype);
  const int CR = chunk_rows_for(p, workspace_bytes, dense);
  if (CR <= 0)
    return fail(PIVOT_ERR_WORKSPACE, "workspace of %zu bytes is below the minimum %zu", workspace_bytes,
                prefill_bytes(p, std::min(p.G, 8), dense));

  hipStream_t s = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  uint8_t* qbar = ws + p.off_qbar;
  float* qbs = (float*)(ws + p.off_qs);
  float* wbar = (float*)(ws + p.off_wbar);
  int32_t* cand = (int32_t*)(ws + p.fixed);
  float* S = (float*)(ws + p.fixed + (dense ? 0 : align_up((size_t)CR * p.m * 4)));
  const uint8_t* qb = (const uint8_t*)q;
  const uint8_t* kb = (const uint8_t*)k;

  if (!dense) {
    ProxyArgs pa{qb, q_scale, w, L, H, D, g, qbar, qbs, wbar};
    PIVOT_LAUNCH_K(PIVOT_K_PROXY, s, launch_proxy_mean(pa, dtype, s), "proxy mean");
  }
  for (int r0 = 0; r0 < p.G; r0 += CR) {
    const int r1 = std::min(p.G, r0 + CR);
    ScanArgs sa{};
    if (dense) {
      sa = ScanArgs{qb, q_scale, w, kb, k_scale, L, H, r0, r1, 1, -excl, L - 1 - excl, kScanKeyChunk, S,
                    p.ldS};
    } else {
      sa = ScanArgs{qbar, qbs, wbar, kb, k_scale, L, H, r0, r1, g, g - 1 - excl, L - 1 - excl, kScanKeyChunk,
                    S, p.ldS};
    }
    // the scan runs in launches of at most kScanRowsPerLaunch rows (measured
    // faster than one launch per pass at 16K-128K, bf16 and fp8)
    for (int rs = r0; rs < r1; rs += kScanRowsPerLaunch) {
      ScanArgs sb = sa;
      sb.row_begin = rs;
      sb.row_end = std::min(r1, rs + kScanRowsPerLaunch);
      sb.S = S + (size_t)(rs - r0) * p.ldS;
      PIVOT_LAUNCH_K(PIVOT_K_SCAN, s, launch_scan(sb, dtype, D, s), "scan");
    }
    TopkArgs ta{};
    ta.S = S;
    ta.ldS = p.ldS;
    ta.row_begin = r0;
    ta.nrows = r1 - r0;
    ta.kind = kLenPos;
    ta.pos_mul = dense ? 1 : g;
    ta.pos_add = (dense ? 0 : g - 1) - excl;
    ta.pos_cap = L - 1 - excl;
    if (dense) {
      ta.m = topk;
      ta.out = out + (size_t)r0 * ldo;
      ta.ldo = ldo;
      if (outs) {
        ta.out_s = outs + (size_t)r0 * topk;
        ta.ldos = topk;
      }
      PIVOT_LAUNCH_K(PIVOT_K_SELECT, s, launch_topk(ta, s), "dense top-k");
      continue;
    }
    int32_t* cdst = cand_user ? cand_user + (size_t)r0 * p.m : cand;
    ta.m = p.m;
    ta.out = cdst;
    ta.ldo = p.m;
    PIVOT_LAUNCH_K(PIVOT_K_SELECT, s, launch_topk(ta, s), "proxy top-m");
    if (cand_user) continue;
    const int row_begin = r0 * g, row_end = std::min(L, r1 * g);
    if (mode == PIVOT_MODE_REUSE) {
      BroadcastArgs ba{cdst, p.m, r0, out + (size_t)row_begin * ldo, topk, 0, g, 0, nullptr,
                       row_begin, row_end, ldo, excl};
      if (outs) {  // the proxy's scores of this pass are still in S
        ba.S = S;
        ba.ldS = p.ldS;
        ba.out_s = outs + (size_t)row_begin * topk;
        ba.ldos = topk;
      }
      PIVOT_LAUNCH_K(PIVOT_K_BROADCAST, s, launch_broadcast(ba, s), "reuse broadcast");
    } else {
      RefineArgs ra{qb, q_scale, w, kb, k_scale, H, 0, L, g, 0, nullptr, r0, r1, cdst, p.m, p.m,
                    kRefineSlotChunk, S, p.ldR, row_begin, excl};
      PIVOT_LAUNCH_K(PIVOT_K_REFINE, s, launch_refine(ra, dtype, D, s), "refine score");
      TopkArgs tr{};
      tr.S = S;
      tr.ldS = p.ldR;
      tr.row_begin = row_begin;
      tr.nrows = row_end - row_begin;
      tr.m = topk;
      tr.out = out + (size_t)row_begin * ldo;
      tr.ldo = ldo;
      tr.excl = excl;
      tr.kind = kLenRefine;
      tr.decode = 0;
      tr.g = g;
      tr.map = cdst;
      tr.ldmap = p.m;
      tr.map_grp_begin = r0;
      if (outs) {
        tr.out_s = outs + (size_t)row_begin * topk;
        tr.ldos = topk;
      }
      PIVOT_LAUNCH_K(PIVOT_K_MEMBER_SELECT, s, launch_topk(tr, s), "refine top-k");
    }
  }
  if (window > 0 && !cand_user) {
    WindowArgs wa{out, ldo, L, topk, window, 0, g, 0, nullptr, 0};
    PIVOT_LAUNCH_K(PIVOT_K_WINDOW, s, launch_window_union(wa, s), "window union");
  }
  return PIVOT_OK;
}

// ---------------------------------------------------------------------------
// Decode plan.
// ---------------------------------------------------------------------------
struct DecodePlan {
  int m;
  int rows;   // scored rows: B proxies, or B*g members for DENSE
  int parts;  // workgroups per row in the decode top-m gather
  int cap;    // keys per gather slice region (a slice never holds more than its length)
  long long ldS, ldR;
  size_t off_qbar, off_qs, off_wbar, off_cand, off_S, off_R, off_hist, off_ckey, off_cslot, off_ccount,
      off_thr, total;
};

DecodePlan plan_decode(int B, int Lmax, int H, int D, int g, int topk, int C, int mode,
                       int dtype) {
  DecodePlan p{};
  const bool dense = mode == PIVOT_MODE_DENSE;
  p.m = mode == PIVOT_MODE_REFINE ? C : topk;
  p.ldS = round_up(Lmax, 64);
  p.ldR = round_up(C, 64);
  size_t off = 0;
  p.off_qbar = off;
  if (!dense) off = align_up(off + (size_t)B * H * D * esize(dtype));
  p.off_qs = off;
  if (!dense) off = align_up(off + (size_t)B * 4);
  p.off_wbar = off;
  if (!dense) off = align_up(off + (size_t)B * H * 4);
  p.off_cand = off;
  if (!dense) off = align_up(off + (size_t)B * p.m * 4);
  p.off_S = off;
  off = align_up(off + (size_t)B * (dense ? g : 1) * p.ldS * 4);
  p.off_R = off;
  if (mode == PIVOT_MODE_REFINE) off = align_up(off + (size_t)B * g * p.ldR * 4);
  p.rows = dense ? B * g : B;
  p.parts = (int)std::min<long long>(32, std::max<long long>(1, (Lmax + 4095) / 4096));
  p.cap = (int)std::min<long long>(kSelectCap, round_up((Lmax + p.parts - 1) / p.parts, 16));
  p.off_hist = off;
  off = align_up(off + (size_t)p.rows * kSelectBins1 * 4);
  p.off_ckey = off;
  off = align_up(off + (size_t)p.rows * p.parts * p.cap * 4);
  p.off_cslot = off;
  off = align_up(off + (size_t)p.rows * p.parts * p.cap * 4);
  p.off_ccount = off;
  off = align_up(off + (size_t)p.rows * p.parts * 4);
  p.off_thr = off;
  off = align_up(off + (size_t)p.rows * 2 * 4);
  p.total = off;
  return p;
}

}  // namespace

extern "C" {

int pivot_version(void) { return 100; }

const char* pivot_status_string(int status) {
  switch (status) {
    case PIVOT_OK: return "ok";
    case PIVOT_ERR_NULL: return "null pointer";
    case PIVOT_ERR_SHAPE: return "invalid shape";
    case PIVOT_ERR_PARAM: return "invalid parameter";
    case PIVOT_ERR_UNSUPPORTED: return "unsupported shape";
    case PIVOT_ERR_ALIGN: return "misaligned pointer";
    case PIVOT_ERR_WORKSPACE: return "workspace too small";
    case PIVOT_ERR_HIP: return "HIP launch failure";
    case PIVOT_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

const char* pivot_last_error_detail(void) { return g_err; }

size_t pivot_workspace_size(int L, int H, int D, int g, int topk, int C, int mode, int dtype) {
  if (L < 1 || H < 1 || D < 1 || g < 1 || topk < 1) return 0;
  const bool dense = mode == PIVOT_MODE_DENSE;
  if (dense) g = 1;
  const PrefillPlan p = plan_prefill(L, H, D, g, topk, C, mode, dtype);
  long long rows = std::max<long long>(8, (long long)(kScoreBudget / p.per_row) / 8 * 8);
  rows = std::min<long long>(rows, p.G);
  return prefill_bytes(p, (int)rows, dense);
}

size_t pivot_workspace_min_size(int L, int H, int D, int g, int topk, int C, int mode, int dtype) {
  if (L < 1 || H < 1 || D < 1 || g < 1 || topk < 1) return 0;
  const bool dense = mode == PIVOT_MODE_DENSE;
  if (dense) g = 1;
  const PrefillPlan p = plan_prefill(L, H, D, g, topk, C, mode, dtype);
  return prefill_bytes(p, std::min(p.G, 8), dense);
}

int pivot_indexer(const void* q, const float* q_scale, const float* w, const void* k,
                  const float* k_scale, int L, int H, int D, int g, int topk, int C, int mode,
                  int dtype, int32_t* out, float* out_scores, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (!out) return fail(PIVOT_ERR_NULL, "out must be non-NULL");
  return run_prefill(q, q_scale, w, k, k_scale, L, H, D, g, topk, C, mode, dtype, out, nullptr,
                     workspace, workspace_bytes, stream, 0, 0, out_scores);
}

// Several sequences run concurrently: each on one of a few library-owned
// streams (default priority, created once per device), each stream with its
// own slice of the workspace, forked from and joined back to the caller's
// stream with events.
constexpr int kVarlenStreams = 4;

size_t pivot_varlen_workspace_size(const int64_t* cu_seqlens, int nseq, int H, int D, int g, int topk,
                                   int C, int mode, int dtype) {
  if (!cu_seqlens || nseq < 1) return 0;
  int Lmax = 0;
  for (int i = 0; i < nseq; ++i) {
    const int64_t n = cu_seqlens[i + 1] - cu_seqlens[i];
    if (n < 0 || n > INT32_MAX) return 0;
    Lmax = std::max<int>(Lmax, (int)n);
  }
  if (Lmax == 0) return 256;
  int nonempty = 0;
  for (int i = 0; i < nseq; ++i) nonempty += cu_seqlens[i + 1] > cu_seqlens[i] ? 1 : 0;
  const size_t slice = align_up(pivot_workspace_size(Lmax, H, D, g, topk, C, mode, dtype));
  return slice * (size_t)std::min(kVarlenStreams, nonempty);
}

namespace {
std::mutex g_vs_mu;
hipStream_t g_vs[kMaxDevices][kVarlenStreams] = {};
bool g_vs_ready[kMaxDevices] = {};

int varlen_streams(hipStream_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(PIVOT_ERR_UNSUPPORTED, "device %d beyond the tracked range", dev);
  std::lock_guard<std::mutex> lk(g_vs_mu);
  if (!g_vs_ready[dev]) {
    for (int k = 0; k < kVarlenStreams; ++k) {
      e = hipStreamCreateWithFlags(&g_vs[dev][k], hipStreamNonBlocking);
      if (e != hipSuccess) return hip_status(e, "hipStreamCreateWithFlags");
    }
    g_vs_ready[dev] = true;
  }
  *out = g_vs[dev];
  return PIVOT_OK;
}
}  // namespace

int pivot_indexer_varlen(const void* q, const float* q_scale, const float* w, const void* k,
                         const float* k_scale, const int64_t* cu_seqlens, int nseq, int H, int D, int g,
                         int topk, int C, int mode, int dtype, int window, int window_mode, int32_t* out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!cu_seqlens) return fail(PIVOT_ERR_NULL, "cu_seqlens must be non-NULL (host memory)");
  if (nseq < 1) return fail(PIVOT_ERR_SHAPE, "nseq=%d must be >= 1", nseq);
  if (cu_seqlens[0] != 0) return fail(PIVOT_ERR_PARAM, "cu_seqlens[0] must be 0");
  for (int i = 0; i < nseq; ++i) {
    const int64_t n = cu_seqlens[i + 1] - cu_seqlens[i];
    if (n < 0 || n > INT32_MAX)
      return fail(PIVOT_ERR_PARAM, "sequence %d has length %lld", i, (long long)n);
  }
  if (!out) return fail(PIVOT_ERR_NULL, "out must be non-NULL");
  // every sequence is checked before anything is enqueued
  int st = validate_common(q, q_scale, w, k, k_scale, H, D, g, topk, C, mode, dtype);
  if (st) return st;
  st = validate_window(window, window_mode, topk);
  if (st) return st;
  if (!workspace) return fail(PIVOT_ERR_NULL, "workspace must be non-NULL");
  if (!aligned(workspace, kAlign)) return fail(PIVOT_ERR_ALIGN, "workspace must be 256-byte aligned");
  const size_t esz = esize(dtype);
  const bool dense = mode == PIVOT_MODE_DENSE;
  std::vector<int> order;
  size_t need_min = 0;  // the largest minimum workspace of any sequence
  for (int i = 0; i < nseq; ++i) {
    const int64_t t0 = cu_seqlens[i];
    const int L = (int)(cu_seqlens[i + 1] - t0);
    if (L == 0) continue;
    const size_t qoff = (size_t)t0 * H * D * esz, koff = (size_t)t0 * D * esz;
    if (!aligned((const uint8_t*)q + qoff, 16) || !aligned((const uint8_t*)k + koff, 16))
      return fail(PIVOT_ERR_ALIGN, "sequence %d: q and k rows must stay 16-byte aligned", i);
    if ((long long)L * D * esz >= (1ll << 31))
      return fail(PIVOT_ERR_SHAPE, "sequence %d: the key array must stay below 2 GiB", i);
    const PrefillPlan p = plan_prefill(L, H, D, dense ? 1 : g, topk, C, mode, dtype);
    need_min = std::max(need_min, prefill_bytes(p, std::min(p.G, 8), dense));
    order.push_back(i);
  }
  if (order.empty()) return PIVOT_OK;
  // slices: as many concurrent sequences as the workspace holds (at least one)
  int nslots = std::min<int>(kVarlenStreams, (int)order.size());
  while (nslots > 1 && (workspace_bytes / nslots) / kAlign * kAlign < need_min) --nslots;
  const size_t slice = nslots > 1 ? (workspace_bytes / nslots) / kAlign * kAlign : workspace_bytes;
  if (slice < need_min)
    return fail(PIVOT_ERR_WORKSPACE, "workspace of %zu bytes is below the minimum %zu", workspace_bytes, need_min);
  auto run_one = [&](int i, void* ws, size_t wsb, void* strm) {
    const int64_t t0 = cu_seqlens[i];
    const int L = (int)(cu_seqlens[i + 1] - t0);
    return run_prefill((const uint8_t*)q + (size_t)t0 * H * D * esz, q_scale ? q_scale + t0 : nullptr,
                       w + (size_t)t0 * H, (const uint8_t*)k + (size_t)t0 * D * esz, k_scale ? k_scale + t0 : nullptr,
                       L, H, D, g, topk, C, mode, dtype, out + (size_t)t0 * (topk + window), nullptr, ws, wsb, strm,
                       window, window_mode);
  };
  if (nslots == 1) {  // one after another on the caller's stream
    for (int i : order)
      if ((st = run_one(i, workspace, workspace_bytes, stream))) return st;
    return PIVOT_OK;
  }
  hipStream_t* pool = nullptr;
  if ((st = varlen_streams(&pool))) return st;
  hipStream_t s = (hipStream_t)stream;
  // longest first, each to the least loaded stream (work ~ L^2)
  std::sort(order.begin(), order.end(), [&](int x, int y) {
    return cu_seqlens[x + 1] - cu_seqlens[x] > cu_seqlens[y + 1] - cu_seqlens[y];
  });
  hipEvent_t fork = nullptr;
  hipError_t e = hipEventCreateWithFlags(&fork, hipEventDisableTiming);
  if (e != hipSuccess) return hip_status(e, "hipEventCreateWithFlags");
  e = hipEventRecord(fork, s);
  for (int j = 0; j < nslots && e == hipSuccess; ++j) e = hipStreamWaitEvent(pool[j], fork, 0);
  (void)hipEventDestroy(fork);
  if (e != hipSuccess) return hip_status(e, "varlen fork");
  std::vector<double> load(nslots, 0.0);
  for (int i : order) {
    const int j = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    const double L = (double)(cu_seqlens[i + 1] - cu_seqlens[i]);
    load[j] += L * L;
    if ((st = run_one(i, (uint8_t*)workspace + (size_t)j * slice, slice, pool[j]))) break;
  }
  // join, also after a failure, so the caller's stream never runs ahead
  for (int j = 0; j < nslots; ++j) {
    hipEvent_t done = nullptr;
    e = hipEventCreateWithFlags(&done, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(done, pool[j]);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, done, 0);
    if (done) (void)hipEventDestroy(done);
    if (e != hipSuccess && st == PIVOT_OK) st = hip_status(e, "varlen join");
  }
  return st;
}

int pivot_candidates(const void* q, const float* q_scale, const float* w, const void* k,
                     const float* k_scale, int L, int H, int D, int g, int topk, int C, int mode,
                     int dtype, int32_t* cand, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (mode == PIVOT_MODE_DENSE)
    return fail(PIVOT_ERR_PARAM, "pivot_candidates needs mode REUSE or REFINE");
  if (!cand) return fail(PIVOT_ERR_NULL, "cand must be non-NULL");
  return run_prefill(q, q_scale, w, k, k_scale, L, H, D, g, topk, C, mode, dtype, nullptr, cand,
                     workspace, workspace_bytes, stream);
}

int pivot_proxy_mean(const void* q, const float* q_scale, const float* w, int L, int H, int D,
                     int g, int dtype, void* qbar, float* qbar_scale, float* wbar, void* stream) {
  int st = validate_common(q, q_scale, w, q, q_scale, H, D, g, 1, 1, PIVOT_MODE_REUSE, dtype);
  if (st) return st;
  if (L < 1) return fail(PIVOT_ERR_SHAPE, "L=%d must be >= 1", L);
  if (!qbar || !qbar_scale || !wbar) return fail(PIVOT_ERR_NULL, "qbar, qbar_scale and wbar must be non-NULL");
  if (!aligned(qbar, 16) || !aligned(qbar_scale, 4) || !aligned(wbar, 4))
    return fail(PIVOT_ERR_ALIGN, "qbar must be 16-byte aligned, qbar_scale and wbar 4-byte aligned");
  ProxyArgs pa{(const uint8_t*)q, q_scale, w, L, H, D, g, (uint8_t*)qbar, qbar_scale, wbar};
  PIVOT_LAUNCH(launch_proxy_mean(pa, dtype, (hipStream_t)stream), "proxy mean");
  return PIVOT_OK;
}

size_t pivot_decode_workspace_size(int B, int Lmax, int H, int D, int g, int topk, int C,
                                   int mode, int dtype) {
  if (B < 1 || Lmax < 1 || H < 1 || D < 1 || g < 1 || topk < 1) return 0;
  return plan_decode(B, Lmax, H, D, g, topk, C, mode, dtype).total + kAlign;
}

// A paged key cache: a pool of num_pages pages of page_size keys (k_cache and
// k_scale point at the pool) and a block table of max_pages page ids per sequence.
struct PagedKeys {
  const int32_t* bt;
  int max_pages, page_size, num_pages;
};

static int validate_pages(const PagedKeys& pk, int D, int dtype) {
  if (!pk.bt) return fail(PIVOT_ERR_NULL, "block_table must be non-NULL");
  if (!aligned(pk.bt, 4)) return fail(PIVOT_ERR_ALIGN, "block_table must be 4-byte aligned");
  if (pk.page_size < 64 || pk.page_size > (1 << 20) || (pk.page_size & (pk.page_size - 1)))
    return fail(PIVOT_ERR_PARAM, "page_size=%d must be a power of two in 64..2^20", pk.page_size);
  if (pk.num_pages < 1 || pk.max_pages < 1)
    return fail(PIVOT_ERR_SHAPE, "num_pages=%d and max_pages=%d must be >= 1", pk.num_pages, pk.max_pages);
  if ((long long)pk.max_pages * pk.page_size > INT32_MAX / 2)
    return fail(PIVOT_ERR_SHAPE, "max_pages * page_size too large");
  if ((long long)pk.num_pages * pk.page_size * D * esize(dtype) >= (1ll << 32))
    return fail(PIVOT_ERR_SHAPE, "the key pool (num_pages * page_size * D codes) must stay below 4 GiB");
  return PIVOT_OK;
}

static void set_pages(DecScanArgs& da, const PagedKeys* pk) {
  if (!pk) return;
  da.bt = pk->bt;
  da.bt_stride = pk->max_pages;
  da.page_shift = __builtin_ctz((unsigned)pk->page_size);
  da.num_pages = pk->num_pages;
}

static int run_decode(const void* q, const float* q_scale, const float* w,
                      const void* k_cache, const float* k_scale, const int32_t* cache_len,
                      int B, int Lmax, int H, int D, int g, int topk, int C, int mode,
                      int dtype, int32_t* out, int32_t* cand_user, void* workspace,
                      size_t workspace_bytes, void* stream, int window = 0, int wmode = 0,
                      const PagedKeys* pk = nullptr, float* outs = nullptr) {
  int st = validate_common(q, q_scale, w, k_cache, k_scale, H, D, g, topk, C, mode, dtype);
  if (st) return st;
  st = validate_window(window, wmode, topk);
  if (st) return st;
  if (pk && (st = validate_pages(*pk, D, dtype))) return st;
  const int excl = wmode == PIVOT_WINDOW_EXCLUDED ? window : 0;
  const long long ldo = (long long)topk + window;
  if (B < 1 || Lmax < 1) return fail(PIVOT_ERR_SHAPE, "B=%d and Lmax=%d must be >= 1", B, Lmax);
  if (g > Lmax) return fail(PIVOT_ERR_PARAM, "g=%d exceeds Lmax=%d", g, Lmax);
  if ((long long)B * Lmax * D > (1ll << 40)) return fail(PIVOT_ERR_SHAPE, "B*Lmax*D too large");
  if ((long long)Lmax * D * esize(dtype) >= (1ll << 31))
    return fail(PIVOT_ERR_SHAPE, "one sequence's key cache (Lmax*D codes) must stay below 2 GiB");
  if (!cache_len || (!out && !cand_user) || !workspace)
    return fail(PIVOT_ERR_NULL, "cache_len, out and workspace must be non-NULL");
  if (!aligned(cache_len, 4) || (out && !aligned(out, 4)) || (cand_user && !aligned(cand_user, 4)) ||
      (outs && !aligned(outs, 4)))
    return fail(PIVOT_ERR_ALIGN, "cache_len and outputs must be 4-byte aligned");
  if (outs && window > 0) return fail(PIVOT_ERR_INTERNAL, "scores are written without a window only");
  if (!aligned(workspace, kAlign)) return fail(PIVOT_ERR_ALIGN, "workspace must be 256-byte aligned");
  const DecodePlan p = plan_decode(B, Lmax, H, D, g, topk, C, mode, dtype);
  if (workspace_bytes < p.total)
    return fail(PIVOT_ERR_WORKSPACE, "workspace of %zu bytes is below the minimum %zu", workspace_bytes, p.total);

  hipStream_t s = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  const uint8_t* qb = (const uint8_t*)q;
  const uint8_t* kb = (const uint8_t*)k_cache;
  float* S = (float*)(ws + p.off_S);

  uint32_t* hist = (uint32_t*)(ws + p.off_hist);
  DecSelectArgs sel{S, p.ldS, p.rows, 0, 0, g, Lmax, cache_len, hist, p.parts,
                    (uint32_t*)(ws + p.off_ckey), (int32_t*)(ws + p.off_cslot), (int32_t*)(ws + p.off_ccount),
                    nullptr, 0, excl};
  sel.thr = (uint32_t*)(ws + p.off_thr);
  sel.cap = p.cap;
  const WindowArgs wa{out, ldo, B * g, topk, window, 1, g, Lmax, cache_len, 0};
  if (mode == PIVOT_MODE_DENSE) {
    PIVOT_LAUNCH_K(PIVOT_K_SELECT, s, launch_fill_u32(hist, (size_t)p.rows * kSelectBins1, 0u, s),
                   "decode histogram clear");
    DecScanArgs da{qb, q_scale, w, kb, k_scale, Lmax, H, cache_len, g, g, S, p.ldS, hist, B, excl};
    set_pages(da, pk);
    PIVOT_LAUNCH_K(PIVOT_K_DECODE_SCAN, s, launch_decode_scan(da, dtype, D, s), "decode scan");
    sel.m = topk;
    sel.kind = kLenDecodeDense;
    sel.out = out;
    sel.ldo = ldo;
    sel.out_s = outs;
    sel.ldos = topk;
    PIVOT_LAUNCH_K(PIVOT_K_SELECT, s, launch_decode_select(sel, s), "decode dense top-k");
    if (window > 0) PIVOT_LAUNCH_K(PIVOT_K_WINDOW, s, launch_window_union(wa, s), "window union");
    return PIVOT_OK;
  }
  uint8_t* qbar = ws + p.off_qbar;
  float* qbs = (float*)(ws + p.off_qs);
  float* wbar = (float*)(ws + p.off_wbar);
  int32_t* cand = cand_user ? cand_user : (int32_t*)(ws + p.off_cand);
  // the proxy kernel also clears the scan's histograms
  ProxyArgs pa{qb, q_scale, w, B * g, H, D, g, qbar, qbs, wbar, hist, (size_t)p.rows * kSelectBins1};
  PIVOT_LAUNCH_K(PIVOT_K_PROXY, s, launch_proxy_mean(pa, dtype, s), "decode proxy mean");
  DecScanArgs da{qbar, qbs, wbar, kb, k_scale, Lmax, H, cache_len, g, 1, S, p.ldS, hist, B, excl};
  set_pages(da, pk);
  PIVOT_LAUNCH_K(PIVOT_K_DECODE_SCAN, s, launch_decode_scan(da, dtype, D, s), "decode scan");
  sel.m = p.m;
  sel.kind = kLenCache;
  sel.out = cand;
  sel.ldo = p.m;
  PIVOT_LAUNCH_K(PIVOT_K_SELECT, s, launch_decode_select(sel, s), "decode proxy top-m");
  if (cand_user) return PIVOT_OK;
  if (mode == PIVOT_MODE_REUSE) {
    BroadcastArgs ba{cand, p.m, 0, out, topk, 1, g, Lmax, cache_len, 0, B * g, ldo, excl};
    if (outs) {
      ba.S = S;
      ba.ldS = p.ldS;
      ba.out_s = outs;
      ba.ldos = topk;
    }
    PIVOT_LAUNCH_K(PIVOT_K_BROADCAST, s, launch_broadcast(ba, s), "decode reuse broadcast");
    if (window > 0) PIVOT_LAUNCH_K(PIVOT_K_WINDOW, s, launch_window_union(wa, s), "window union");
    return PIVOT_OK;
  }
  float* R = (float*)(ws + p.off_R);
  RefineArgs ra{qb, q_scale, w, kb, k_scale, H, 1, 0, g, Lmax, cache_len, 0, B, cand, p.m, p.m,
                kRefineSlotChunk, R, p.ldR, 0, excl};
  if (pk) {
    ra.bt = pk->bt;
    ra.bt_stride = pk->max_pages;
    ra.page_shift = __builtin_ctz((unsigned)pk->page_size);
    ra.pool_rows = pk->num_pages * pk->page_size;
  }
  PIVOT_LAUNCH_K(PIVOT_K_REFINE, s, launch_refine(ra, dtype, D, s), "decode refine score");
  TopkArgs tr{};
  tr.S = R;
  tr.ldS = p.ldR;
  tr.row_begin = 0;
  tr.nrows = B * g;
  tr.m = topk;
  tr.out = out;
  tr.ldo = ldo;
  tr.excl = excl;
  tr.kind = kLenRefine;
  tr.decode = 1;
  tr.g = g;
  tr.Lmax = Lmax;
  tr.cache_len = cache_len;
  tr.map = cand;
  tr.ldmap = p.m;
  tr.map_grp_begin = 0;
  tr.out_s = outs;
  tr.ldos = topk;
  PIVOT_LAUNCH_K(PIVOT_K_MEMBER_SELECT, s, launch_topk(tr, s), "decode refine top-k");
  if (window > 0) PIVOT_LAUNCH_K(PIVOT_K_WINDOW, s, launch_window_union(wa, s), "window union");
  return PIVOT_OK;
}

int pivot_indexer_decode(const void* q, const float* q_scale, const float* w,
                         const void* k_cache, const float* k_scale, const int32_t* cache_len,
                         int B, int Lmax, int H, int D, int g, int topk, int C, int mode,
                         int dtype, int32_t* out, float* out_scores, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!out) return fail(PIVOT_ERR_NULL, "out must be non-NULL");
  return run_decode(q, q_scale, w, k_cache, k_scale, cache_len, B, Lmax, H, D, g, topk, C, mode,
                    dtype, out, nullptr, workspace, workspace_bytes, stream, 0, 0, nullptr, out_scores);
}

int pivot_indexer_window(const void* q, const float* q_scale, const float* w, const void* k,
                         const float* k_scale, int L, int H, int D, int g, int topk, int C,
                         int mode, int dtype, int window, int window_mode, int32_t* out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!out) return fail(PIVOT_ERR_NULL, "out must be non-NULL");
  return run_prefill(q, q_scale, w, k, k_scale, L, H, D, g, topk, C, mode, dtype, out, nullptr,
                     workspace, workspace_bytes, stream, window, window_mode);
}

int pivot_indexer_decode_window(const void* q, const float* q_scale, const float* w,
                                const void* k_cache, const float* k_scale, const int32_t* cache_len,
                                int B, int Lmax, int H, int D, int g, int topk, int C, int mode,
                                int dtype, int window, int window_mode, int32_t* out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!out) return fail(PIVOT_ERR_NULL, "out must be non-NULL");
  return run_decode(q, q_scale, w, k_cache, k_scale, cache_len, B, Lmax, H, D, g, topk, C, mode,
                    dtype, out, nullptr, workspace, workspace_bytes, stream, window, window_mode);
}

int pivot_indexer_decode_paged(const void* q, const float* q_scale, const float* w, const void* k_pages,
                               const float* k_scale_pages, int num_pages, int page_size,
                               const int32_t* block_table, int max_pages, const int32_t* cache_len, int B,
                               int H, int D, int g, int topk, int C, int mode, int dtype, int window,
                               int window_mode, int32_t* out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!out) return fail(PIVOT_ERR_NULL, "out must be non-NULL");
  const PagedKeys pk{block_table, max_pages, page_size, num_pages};
  int st = validate_pages(pk, D, dtype);
  if (st) return st;
  return run_decode(q, q_scale, w, k_pages, k_scale_pages, cache_len, B, max_pages * page_size, H, D, g, topk, C,
                    mode, dtype, out, nullptr, workspace, workspace_bytes, stream, window, window_mode, &pk);
}

// ---------------------------------------------------------------------------
// Allocation-free decode step.  Its scratch memory is this device array (one
// copy per GPU, held until the process ends); host code only ever uses the
// device address hipGetSymbolAddress returns for the current GPU.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the current device (looked up once per device).
int scratch_of_current_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PIVOT_ERR_UNSUPPORTED, "device %d: the allocation-free entry point tracks devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(PIVOT_ERR_INTERNAL, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PIVOT_OK;
}
}  // namespace

int pivot_indexer_decode_noalloc(const void* q, const float* q_scale, const float* w, const void* k_cache,
                                 const float* k_scale, const int32_t* cache_len, int B, int Lmax, int H, int D,
                                 int g, int topk, int C, int mode, int dtype, int32_t* out, float* out_scores,
                                 void* stream) {
  if (!out) return fail(PIVOT_ERR_NULL, "out must be non-NULL");
  void* ws = nullptr;
  int st = scratch_of_current_device(&ws);
  if (st) return st;
  st = run_decode(q, q_scale, w, k_cache, k_scale, cache_len, B, Lmax, H, D, g, topk, C, mode, dtype, out,
                  nullptr, ws, kNoAllocScratchBytes, stream, 0, 0, nullptr, out_scores);
  if (st == PIVOT_ERR_WORKSPACE)
    return fail(PIVOT_ERR_WORKSPACE,
                "this decode step needs %zu bytes of scratch; the allocation-free entry point holds %zu",
                pivot_decode_workspace_size(B, Lmax, H, D, g, topk, C, mode, dtype), kNoAllocScratchBytes);
  return st;
}

size_t pivot_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int pivot_decode_candidates(const void* q, const float* q_scale, const float* w,
                            const void* k_cache, const float* k_scale, const int32_t* cache_len,
                            int B, int Lmax, int H, int D, int g, int topk, int C, int mode,
                            int dtype, int32_t* cand, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (mode == PIVOT_MODE_DENSE)
    return fail(PIVOT_ERR_PARAM, "pivot_decode_candidates needs mode REUSE or REFINE");
  if (!cand) return fail(PIVOT_ERR_NULL, "cand must be non-NULL");
  return run_decode(q, q_scale, w, k_cache, k_scale, cache_len, B, Lmax, H, D, g, topk, C, mode,
                    dtype, nullptr, cand, workspace, workspace_bytes, stream);
}

int pivot_dbg_score_rows(const void* q, const float* q_scale, const float* w, const void* k,
                         const float* k_scale, int R, int Lk, int H, int D, int dtype, int row_begin,
                         int row_end, int pos_mul, int pos_add, float* S, long long ldS, void* stream) {
  int st = validate_common(q, q_scale, w, k, k_scale, H, D, 1, 1, 1, PIVOT_MODE_DENSE, dtype);
  if (st) return st;
  if (R < 1 || Lk < 1) return fail(PIVOT_ERR_SHAPE, "R=%d and Lk=%d must be >= 1", R, Lk);
  if ((long long)Lk * D * esize(dtype) >= (1ll << 31))
    return fail(PIVOT_ERR_SHAPE, "the key array (Lk*D codes) must stay below 2 GiB");
  if (row_begin < 0 || row_end > R || row_begin > row_end)
    return fail(PIVOT_ERR_SHAPE, "rows [%d, %d) must lie in [0, %d)", row_begin, row_end, R);
  if (pos_mul < 0) return fail(PIVOT_ERR_PARAM, "pos_mul=%d must be >= 0", pos_mul);
  if (!S) return fail(PIVOT_ERR_NULL, "S must be non-NULL");
  if (!aligned(S, 4)) return fail(PIVOT_ERR_ALIGN, "S must be 4-byte aligned");
  if (row_begin == row_end) return PIVOT_OK;
  const long long plast = std::min<long long>((long long)(row_end - 1) * pos_mul + pos_add, Lk - 1);
  if (ldS < plast + 1) return fail(PIVOT_ERR_PARAM, "ldS=%lld is below the last row's %lld scores", ldS, plast + 1);
  if ((long long)row_end * pos_mul + pos_add > INT32_MAX)
    return fail(PIVOT_ERR_PARAM, "row positions overflow");
  hipStream_t s = (hipStream_t)stream;
  const ScanArgs sa{(const uint8_t*)q, q_scale, w, (const uint8_t*)k, k_scale, Lk, H, row_begin, row_end,
                    pos_mul, pos_add, Lk - 1, kScanKeyChunk, S, ldS};
  for (int rs = row_begin; rs < row_end; rs += kScanRowsPerLaunch) {
    ScanArgs sb = sa;
    sb.row_begin = rs;
    sb.row_end = std::min(row_end, rs + kScanRowsPerLaunch);
    sb.S = S + (size_t)(rs - row_begin) * ldS;
    PIVOT_LAUNCH_K(PIVOT_K_SCAN, s, launch_scan(sb, dtype, D, s), "score rows");
  }
  return PIVOT_OK;
}

// ---------------------------------------------------------------------------
// Cross-layer index reuse stacked on the indexer: full layers run the indexer
// on their own inputs, every other layer takes the rows of the nearest full
// layer before it.
// ---------------------------------------------------------------------------
// Prefixes the last message with the failing layer.
static int layer_fail(int st, int layer) {
  char prev[sizeof g_err];
  snprintf(prev, sizeof prev, "%s", g_err);
  return fail(st, "layer %d: %s", layer, prev);
}

static int validate_layers(int nlayers, const int32_t* full, const void* const* arrays[], int narrays,
                           int32_t* const* out) {
  if (nlayers < 1) return fail(PIVOT_ERR_SHAPE, "nlayers=%d must be >= 1", nlayers);
  if (!full || !out) return fail(PIVOT_ERR_NULL, "full and out must be non-NULL (host arrays)");
  for (int a = 0; a < narrays; ++a)
    if (!arrays[a]) return fail(PIVOT_ERR_NULL, "the per-layer pointer arrays must be non-NULL (host arrays)");
  if (!full[0]) return fail(PIVOT_ERR_PARAM, "layer 0 must run its indexer (full[0] != 0)");
  for (int l = 0; l < nlayers; ++l)
    if (!out[l]) return fail(PIVOT_ERR_NULL, "out[%d] must be non-NULL", l);
  return PIVOT_OK;
}

static int copy_layer(int32_t* const* out, int l, int src, size_t n, hipStream_t s) {
  if (out[l] == out[src]) return PIVOT_OK;  // the caller aliased the rows
  PIVOT_LAUNCH_K(PIVOT_K_LAYER_COPY, s, launch_copy_i32(out[src], out[l], n, s), "layer index copy");
  return PIVOT_OK;
}

int pivot_indexer_layers(int nlayers, const int32_t* full, const void* const* q, const float* const* q_scale,
                         const float* const* w, const void* const* k, const float* const* k_scale, int L, int H,
                         int D, int g, int topk, int C, int mode, int dtype, int32_t* const* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  const void* const* arrays[] = {(const void* const*)q, (const void* const*)w, (const void* const*)k};
  int st = validate_layers(nlayers, full, arrays, 3, out);
  if (st) return st;
  if (dtype == PIVOT_FP8_E4M3 && (!q_scale || !k_scale))
    return fail(PIVOT_ERR_NULL, "fp8 layers need q_scale and k_scale arrays");
  // every full layer is checked before anything is enqueued
  for (int l = 0; l < nlayers; ++l) {
    if (!full[l]) continue;
    st = validate_common(q[l], q_scale ? q_scale[l] : nullptr, w[l], k[l], k_scale ? k_scale[l] : nullptr, H, D, g,
                         topk, C, mode, dtype);
    if (st) return layer_fail(st, l);
  }
  hipStream_t s = (hipStream_t)stream;
  int src = 0;
  for (int l = 0; l < nlayers; ++l) {
    if (full[l]) {
      src = l;
      st = run_prefill(q[l], q_scale ? q_scale[l] : nullptr, w[l], k[l], k_scale ? k_scale[l] : nullptr, L, H, D, g,
                       topk, C, mode, dtype, out[l], nullptr, workspace, workspace_bytes, stream);
      if (st) return st;
    } else if ((st = copy_layer(out, l, src, (size_t)L * topk, s))) {
      return st;
    }
  }
  return PIVOT_OK;
}

int pivot_indexer_decode_layers(int nlayers, const int32_t* full, const void* const* q, const float* const* q_scale,
                                const float* const* w, const void* const* k_cache, const float* const* k_scale,
                                const int32_t* cache_len, int B, int Lmax, int H, int D, int g, int topk, int C,
                                int mode, int dtype, int32_t* const* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  const void* const* arrays[] = {(const void* const*)q, (const void* const*)w, (const void* const*)k_cache};
  int st = validate_layers(nlayers, full, arrays, 3, out);
  if (st) return st;
  if (dtype == PIVOT_FP8_E4M3 && (!q_scale || !k_scale))
    return fail(PIVOT_ERR_NULL, "fp8 layers need q_scale and k_scale arrays");
  for (int l = 0; l < nlayers; ++l) {
    if (!full[l]) continue;
    st = validate_common(q[l], q_scale ? q_scale[l] : nullptr, w[l], k_cache[l], k_scale ? k_scale[l] : nullptr, H,
                         D, g, topk, C, mode, dtype);
    if (st) return layer_fail(st, l);
  }
  hipStream_t s = (hipStream_t)stream;
  int src = 0;
  for (int l = 0; l < nlayers; ++l) {
    if (full[l]) {
      src = l;
      st = run_decode(q[l], q_scale ? q_scale[l] : nullptr, w[l], k_cache[l], k_scale ? k_scale[l] : nullptr,
                      cache_len, B, Lmax, H, D, g, topk, C, mode, dtype, out[l], nullptr, workspace, workspace_bytes,
                      stream);
      if (st) return st;
    } else if ((st = copy_layer(out, l, src, (size_t)B * g * topk, s))) {
      return st;
    }
  }
  return PIVOT_OK;
}

// Sparse main attention: chunks per row.  Many rows: one chunk each (no
// merge); few rows: chunks of at least kSAttnChunk slots, as many as bring the
// launch to about kSAttnTargetWGs workgroups (512 measured about 3 % faster
// than 1024 for the 64 decode rows of 2048 slots, 256 slower).
constexpr int kSAttnChunk = 128;
constexpr int kSAttnTargetWGs = 512;

static void sattn_plan(int R, int nidx, int* chunk, int* nch) {
  const int slots = (nidx + 31) / 32 * 32;
  if ((long long)R >= 1024 || nidx <= kSAttnChunk) {
    *chunk = std::max(32, slots);
    *nch = 1;
    return;
  }
  const int want = std::max(1, std::min((kSAttnTargetWGs + R - 1) / R, (slots + kSAttnChunk - 1) / kSAttnChunk));
  *chunk = (slots / want + 31) / 32 * 32;
  *nch = (nidx + *chunk - 1) / *chunk;
}

size_t pivot_sparse_attention_workspace_size(int R, int Hq, int dv, int nidx) {
  if (R < 1 || Hq < 1 || dv < 1 || nidx < 1) return 0;
  int chunk, nch;
  sattn_plan(R, nidx, &chunk, &nch);
  if (nch == 1) return 0;
  return align_up((size_t)R * nch * Hq * dv * 4) + align_up((size_t)R * nch * 2 * Hq * 4);
}

int pivot_sparse_attention(const void* q, const void* k, const void* v, const int32_t* idx, int R,
                           int Hq, int d, int dv, int nidx, int rows_per_seq, long long seq_stride,
                           int seq_len, float scale, float* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !idx || !out) return fail(PIVOT_ERR_NULL, "q, k, v, idx and out must be non-NULL");
  if (R < 1 || nidx < 1) return fail(PIVOT_ERR_SHAPE, "R=%d and nidx=%d must be >= 1", R, nidx);
  if (!sattn_shape_supported(Hq, d, dv))
    return fail(PIVOT_ERR_UNSUPPORTED, "sparse attention supports d = dv = 128 and Hq in {32, 64} (got %d, %d, %d)", d,
                dv, Hq);
  if (rows_per_seq < 1 || seq_len < 0 || seq_stride < 0)
    return fail(PIVOT_ERR_PARAM, "rows_per_seq=%d must be >= 1, seq_len=%d and seq_stride=%lld >= 0", rows_per_seq,
                seq_len, seq_stride);
  if ((R - 1) / rows_per_seq > 0 && seq_stride < seq_len)
    return fail(PIVOT_ERR_PARAM, "seq_stride=%lld is below seq_len=%d with several sequences", seq_stride, seq_len);
  // below 2 GiB: row offsets fit a signed 32-bit product, and the offset the
  // gathers use for skipped entries lies past every buffer's range
  if ((long long)seq_len * std::max(d, dv) * 2 >= (1ll << 31))
    return fail(PIVOT_ERR_SHAPE, "one sequence's key or value rows must stay below 2 GiB");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(PIVOT_ERR_PARAM, "scale must be finite and > 0");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(idx, 4))
    return fail(PIVOT_ERR_ALIGN, "q, k, v and out must be 16-byte aligned, idx 4-byte aligned");
  int chunk, nch;
  sattn_plan(R, nidx, &chunk, &nch);
  const size_t need = pivot_sparse_attention_workspace_size(R, Hq, dv, nidx);
  if (need > 0) {
    if (!workspace) return fail(PIVOT_ERR_NULL, "workspace must be non-NULL (%zu bytes)", need);
    if (!aligned(workspace, kAlign)) return fail(PIVOT_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(PIVOT_ERR_WORKSPACE, "workspace of %zu bytes is below the minimum %zu", workspace_bytes, need);
  }
  uint8_t* ws = (uint8_t*)workspace;
  SAttnArgs a{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, idx, R, Hq, nidx, rows_per_seq,
              seq_stride, seq_len, scale, chunk, nch, out,
              need ? (float*)ws : nullptr,
              need ? (float*)(ws + align_up((size_t)R * nch * Hq * dv * 4)) : nullptr};
  hipStream_t s = (hipStream_t)stream;
  PIVOT_LAUNCH_K(PIVOT_K_ATTENTION, s, launch_sparse_attention(a, s), "sparse attention");
  return PIVOT_OK;
}

int pivot_profile_enable(int on) {
  g_prof_on.store(on != 0);
  return PIVOT_OK;
}

int pivot_profile_read(double* ms, long long* launches, int n) {
  if ((!ms || !launches) && n > 0) return fail(PIVOT_ERR_NULL, "ms and launches must be non-NULL");
  for (int i = 0; i < n; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  std::vector<TimedLaunch> rec;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    rec.swap(g_prof);
  }
  int st = PIVOT_OK;
  for (const TimedLaunch& t : rec) {
    float el = 0.f;
    hipError_t e = hipEventSynchronize(t.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&el, t.start, t.stop);
    if (e != hipSuccess && st == PIVOT_OK) st = hip_status(e, "profile read");
    if (t.cls < n) {
      ms[t.cls] += el;
      launches[t.cls] += 1;
    }
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  return st;
}

int pivot_selftest_mfma_layout(int32_t* out, void* stream) {
  if (!out) return fail(PIVOT_ERR_NULL, "out must be non-NULL");
  PIVOT_LAUNCH(launch_selftest_mfma(out, (hipStream_t)stream), "mfma self-test");
  return PIVOT_OK;
}

}  // extern "C"
