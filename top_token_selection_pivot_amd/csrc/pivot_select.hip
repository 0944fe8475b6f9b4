// pivot_select.hip -- proxy mean, top-m selection, Reuse broadcast and the
// matrix-core layout self-test (gfx950).
#include <algorithm>

#include "pivot_device.h"
#include "pivot_kernels.h"
#include "pivot_select.h"

namespace pivot {

hipError_t launch_scan_bf16(const ScanArgs&, int, hipStream_t);
hipError_t launch_scan_fp8(const ScanArgs&, int, hipStream_t);
hipError_t launch_refine_bf16(const RefineArgs&, int, hipStream_t);
hipError_t launch_refine_fp8(const RefineArgs&, int, hipStream_t);
hipError_t launch_decode_scan_bf16(const DecScanArgs&, int, hipStream_t);
hipError_t launch_decode_scan_fp8(const DecScanArgs&, int, hipStream_t);

hipError_t launch_scan(const ScanArgs& a, int dtype, int D, hipStream_t st) {
  return dtype == kBF16 ? launch_scan_bf16(a, D, st) : launch_scan_fp8(a, D, st);
}
hipError_t launch_refine(const RefineArgs& a, int dtype, int D, hipStream_t st) {
  return dtype == kBF16 ? launch_refine_bf16(a, D, st) : launch_refine_fp8(a, D, st);
}
hipError_t launch_decode_scan(const DecScanArgs& a, int dtype, int D, hipStream_t st) {
  return dtype == kBF16 ? launch_decode_scan_bf16(a, D, st)
                        : launch_decode_scan_fp8(a, D, st);
}

bool score_shape_supported(int dtype, int D) {
  if (dtype == kBF16) return D == 32 || D == 64 || D == 128 || D == 256;
  return D == 64 || D == 128 || D == 256;
}

// ---------------------------------------------------------------------------
// Proxy mean (molayo1419.me "PIVOT explained", How It Works: the proxy is the
// mean of its group; arXiv:2607.24593 abstract).  One workgroup per group.
// The binary32 sum runs over members in ascending position with no fused
// multiply-add, then one correctly rounded division by the member count.
// ---------------------------------------------------------------------------
constexpr int kProxyThreads = 512;
constexpr int kProxyChunk = 16;                                  // elements per 16-element chunk
constexpr int kProxyMaxCPT = 64 * 256 / kProxyChunk / kProxyThreads;  // chunks per thread (H*D <= 16384)
constexpr int kProxyU = 4;  // members whose loads are issued together

// Chunk c of row `row` as loaded (16 codes; the row scale for fp8) ...
struct ChunkRaw {
  i32x4 lo, hi;  // bf16: 8 + 8 codes; fp8: lo holds all 16 codes
  float s;
};
template <int DT>
__device__ inline ChunkRaw chunk_load(const ProxyArgs& a, int row, int c) {
  const size_t HD = (size_t)a.H * a.D;
  ChunkRaw r;
  if constexpr (DT == kBF16) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(a.q) + (size_t)row * HD + (size_t)c * kProxyChunk;
    r.lo = *reinterpret_cast<const i32x4*>(p);
    r.hi = *reinterpret_cast<const i32x4*>(p + 8);
    r.s = 1.f;
  } else {
    r.lo = *reinterpret_cast<const i32x4*>(a.q + (size_t)row * HD + (size_t)c * kProxyChunk);
    r.hi = r.lo;
    r.s = a.q_scale[row];
  }
  return r;
}
// ... and its 16 values (binary32; fp8 codes times the row scale).
template <int DT>
__device__ inline void chunk_values(const ChunkRaw& r, float* x) {
  if constexpr (DT == kBF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e + 0] = __uint_as_float((uint32_t)r.lo[e] << 16);
      x[2 * e + 1] = __uint_as_float((uint32_t)r.lo[e] & 0xFFFF0000u);
      x[8 + 2 * e + 0] = __uint_as_float((uint32_t)r.hi[e] << 16);
      x[8 + 2 * e + 1] = __uint_as_float((uint32_t)r.hi[e] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // exact decode (hardware E4M3FN conversion)
      x[4 * q + 0] = __fmul_rn(r.s, __builtin_amdgcn_cvt_f32_fp8(r.lo[q], 0));
      x[4 * q + 1] = __fmul_rn(r.s, __builtin_amdgcn_cvt_f32_fp8(r.lo[q], 1));
      x[4 * q + 2] = __fmul_rn(r.s, __builtin_amdgcn_cvt_f32_fp8(r.lo[q], 2));
      x[4 * q + 3] = __fmul_rn(r.s, __builtin_amdgcn_cvt_f32_fp8(r.lo[q], 3));
    }
  }
}

template <int DT>
__global__ __launch_bounds__(kProxyThreads) void proxy_mean_kernel(ProxyArgs a) {
  const int j = blockIdx.x, tid = threadIdx.x;
  for (size_t e = (size_t)j * kProxyThreads + tid; e < a.nzero; e += (size_t)gridDim.x * kProxyThreads)
    a.zero[e] = 0u;
  const int r0 = j * a.g;
  const int n = min(a.g, a.R - r0);
  const size_t HD = (size_t)a.H * a.D;
  const int nch = (int)(HD / kProxyChunk);
  if (n == 1) {  // a one-member group is its member
    const size_t bytes = HD * (DT == kBF16 ? 2 : 1);
    for (size_t e = (size_t)tid * 16; e < bytes; e += (size_t)kProxyThreads * 16)
      *reinterpret_cast<i32x4*>(a.qbar + j * bytes + e) = *reinterpret_cast<const i32x4*>(a.q + (size_t)r0 * bytes + e);
    if (tid == 0) a.qbar_scale[j] = DT == kBF16 ? 1.f : a.q_scale[r0];
    for (int h = tid; h < a.H; h += kProxyThreads) a.wbar[(size_t)j * a.H + h] = a.w[(size_t)r0 * a.H + h];
    return;
  }
  // With a power-of-two member count the division is a product with 1/n:
  // both round the same exact quotient once, so the result is identical.
  const bool pow2 = (n & (n - 1)) == 0;
  const float inv_n = __uint_as_float((uint32_t)(127 - __builtin_ctz((unsigned)n)) << 23);  // 2^-log2(n)
  auto mean_of = [&](float sum) { return pow2 ? sum * inv_n : __fdiv_rn(sum, (float)n); };
  // Members are read kProxyU at a time so that their loads are in flight
  // together (past the last member the load repeats it and is not used; for
  // the weights +0 is added instead, which leaves a running sum unchanged: a
  // sum that starts at +0 is never -0).
  for (int h = tid; h < a.H; h += kProxyThreads) {
    float s = 0.f;
    for (int t0 = 0; t0 < n; t0 += kProxyU) {
      float x[kProxyU];
#pragma unroll
      for (int u = 0; u < kProxyU; ++u) x[u] = a.w[(size_t)(r0 + min(t0 + u, n - 1)) * a.H + h];
#pragma unroll
      for (int u = 0; u < kProxyU; ++u) s = __fadd_rn(s, t0 + u < n ? x[u] : 0.f);
    }
    a.wbar[(size_t)j * a.H + h] = mean_of(s);
  }
  // means of this thread's chunks, members added in ascending position
  float mean[kProxyMaxCPT][kProxyChunk];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kProxyMaxCPT; ++i) {
    const int c = tid + i * kProxyThreads;
    if (c >= nch) continue;
    float acc[kProxyChunk];
#pragma unroll
    for (int e = 0; e < kProxyChunk; ++e) acc[e] = 0.f;
    for (int t0 = 0; t0 < n; t0 += kProxyU) {
      ChunkRaw raw[kProxyU];
#pragma unroll
      for (int u = 0; u < kProxyU; ++u) raw[u] = chunk_load<DT>(a, r0 + min(t0 + u, n - 1), c);
#pragma unroll
      for (int u = 0; u < kProxyU; ++u) {
        if (t0 + u >= n) break;
        float x[kProxyChunk];
        chunk_values<DT>(raw[u], x);
#pragma unroll
        for (int e = 0; e < kProxyChunk; ++e) acc[e] = __fadd_rn(acc[e], x[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < kProxyChunk; ++e) {
      mean[i][e] = mean_of(acc[e]);
      amax = fmaxf(amax, fabsf(mean[i][e]));
    }
  }
  if constexpr (DT == kBF16) {
#pragma unroll
    for (int i = 0; i < kProxyMaxCPT; ++i) {
      const int c = tid + i * kProxyThreads;
      if (c >= nch) continue;
      uint32_t w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        w[e] = (uint32_t)f32_to_bf16_rne(mean[i][2 * e]) | ((uint32_t)f32_to_bf16_rne(mean[i][2 * e + 1]) << 16);
      uint16_t* out = reinterpret_cast<uint16_t*>(a.qbar) + (size_t)j * HD + (size_t)c * kProxyChunk;
      *reinterpret_cast<i32x4*>(out) = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      *reinterpret_cast<i32x4*>(out + 8) = i32x4{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
    }
    if (tid == 0) a.qbar_scale[j] = 1.f;
  } else {
    __shared__ float red[kProxyThreads / kWave];
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = red[0];
    for (int i = 1; i < kProxyThreads / kWave; ++i) amax = fmaxf(amax, red[i]);
    const float sp = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
#pragma unroll
    for (int i = 0; i < kProxyMaxCPT; ++i) {
      const int c = tid + i * kProxyThreads;
      if (c >= nch) continue;
      // E4M3FN codes, round to nearest even, saturating at +-448: the
      // hardware conversion of the value clamped to +-448
      auto sat = [](float v) { return fminf(fmaxf(v, -448.f), 448.f); };
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float* v = &mean[i][4 * q];
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(sat(__fdiv_rn(v[0], sp)), sat(__fdiv_rn(v[1], sp)), 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(sat(__fdiv_rn(v[2], sp)), sat(__fdiv_rn(v[3], sp)), pk, true);
        w[q] = (uint32_t)pk;
      }
      *reinterpret_cast<i32x4*>(a.qbar + (size_t)j * HD + (size_t)c * kProxyChunk) =
          i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
    if (tid == 0) a.qbar_scale[j] = sp;
  }
}

hipError_t launch_proxy_mean(const ProxyArgs& a, int dtype, hipStream_t st) {
  const int G = (a.R + a.g - 1) / a.g;
  if (dtype == kBF16)
    hipLaunchKernelGGL(proxy_mean_kernel<kBF16>, dim3(G), dim3(kProxyThreads), 0, st, a);
  else
    hipLaunchKernelGGL(proxy_mean_kernel<kFP8>, dim3(G), dim3(kProxyThreads), 0, st, a);
  return hipGetLastError();
}

template <int NT>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
  constexpr int NB1 = 1 << kTopkBits1;
  __shared__ SelectShared sm;

  const int tid = threadIdx.x;
  const int i = blockIdx.x;
  const int R = a.row_begin + i;
  const float* row = a.S + (long long)i * a.ldS;
  int32_t* out = a.out + (long long)i * a.ldo;
  float* outs = a.out_s ? a.out_s + (long long)i * a.ldos : nullptr;
  const bool whole_pre = a.kind == kLenRefine && a.ldmap <= kTopkU * NT * 4;
  for (int b = tid; b < NB1; b += NT) sm.hist[b] = 0u;
  // a Refine row has at most ldmap scores: when they fit one pass-1 round
  // they are loaded while the row length is still being counted
  float4 v[kTopkU];
  if (whole_pre) {
#pragma unroll
    for (int u = 0; u < kTopkU; ++u) v[u] = load4(row, (u * NT + tid) * 4, a.ldmap);
  }
  const int32_t* list;
  int n;
  if (a.kind == kLenRefine) {
    // the entries of the ascending, -1 padded candidate list that are <= the
    // member's position, counted in one coalesced pass
    int t;
    n = refine_row_list(a, R, &list, &t);
    if (list) {
      uint32_t c = 0;
      for (int e = tid; e < a.ldmap; e += NT) {
        const int v = list[e];
        c += (v >= 0 && v <= t) ? 1u : 0u;
      }
      uint32_t tot;
      block_exclusive_sum<NT>(c, sm.scratch, &tot);
      n = (int)tot;
    }
  } else {
    n = row_length(a, R, &list);
  }
  const uint32_t m = (uint32_t)a.m;

  if (n <= (int)m) {
    for (int s = tid; s < (int)m; s += NT) {
      out[s] = s < n ? (list ? list[s] : s) : -1;
      if (outs) outs[s] = s < n ? row[s] : no_score();
    }
    return;
  }

  // ---- pass 1: histogram of the top 12 bits (rows that fit are staged in LDS)
  const bool whole = n <= kTopkCap;
  // A long row is first sampled (the first 64 scores of every 1024): the bin
  // holding a conservative rank of the sample, b_est, is at or below the
  // row's threshold bin unless the sample is far off.  Pass 1 then histograms
  // and gathers into LDS, in index order, only the keys whose first digit is
  // >= b_est.  With at least m of them the threshold bin b1 is >= b_est and
  // the histogram of those bins finds it; if they also fit, the row has been
  // read once, else pass 2 gathers from the row.  With fewer than m the
  // whole row is histogrammed again.
  const bool est = !whole && n >= kTopkSampleMin;
  uint32_t b_est = NB1;
  __syncthreads();
  if (est) {
    const int nch = n >> 10;  // whole chunks of 1024 scores
    for (int i = tid; i < nch * 16; i += NT) {
      const float4 s4 = *reinterpret_cast<const float4*>(row + ((i >> 4) << 10) + ((i & 15) << 2));
#pragma unroll
      for (int e = 0; e < 4; ++e) atomicAdd(&sm.hist[score_key(f4(s4, e)) >> (32 - kTopkBits1)], 1u);
    }
    __syncthreads();
    const uint32_t ns = (uint32_t)nch * 64u;
    const float r = (float)m * (float)ns / (float)n;  // the threshold's expected rank in the sample
    const uint32_t rank = (uint32_t)(r + 3.f * sqrtf(r)) + 2u;
    b_est = 0u;
    if (rank <= ns) {
      find_bin<NT>(sm.hist, NB1, rank, sm.scratch, &sm.sh_bin, &sm.sh_above);
      b_est = sm.sh_bin;
    }
    for (int b = tid; b < NB1; b += NT) sm.hist[b] = 0u;
    __syncthreads();
  }
  uint32_t gathered = 0;  // keys with first digit >= b_est (staged while they fit)
  if (est) {
    // rounds of 16 consecutive scores per thread; the next round's loads are
    // in flight during this round's block scan
    constexpr int E = 4 * kTopkU;
    float4 nx[kTopkU];
#pragma unroll
    for (int u = 0; u < kTopkU; ++u) nx[u] = load4(row, tid * E + 4 * u, n);
    for (int base = 0; base < n; base += E * NT) {
      const int s0 = base + tid * E;
      float4 v4[kTopkU];
#pragma unroll
      for (int u = 0; u < kTopkU; ++u) v4[u] = nx[u];
      if (base + E * NT < n) {
#pragma unroll
        for (int u = 0; u < kTopkU; ++u) nx[u] = load4(row, s0 + E * NT + 4 * u, n);
      }
      uint32_t key[E];
      uint32_t cnt = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        key[e] = score_key(f4(v4[e >> 2], e & 3));
        if (s0 + e < n && (key[e] >> (32 - kTopkBits1)) >= b_est) {
          atomicAdd(&sm.hist[key[e] >> (32 - kTopkBits1)], 1u);
          ++cnt;
        }
      }
      uint32_t tot;
      uint32_t p = gathered + block_exclusive_sum<NT>(cnt, sm.scratch, &tot);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (s0 + e < n && (key[e] >> (32 - kTopkBits1)) >= b_est) {
          if (p < (uint32_t)kTopkCap) {
            sm.ckey[p] = key[e];
            sm.cslot[p] = s0 + e;
          }
          ++p;
        }
      }
      gathered += tot;
    }
  }
  // the full first-digit histogram: rows that were not sampled, and sampled
  // rows whose estimate was above the threshold bin
  const bool full = !est || gathered < m;
  if (est && full) {
    __syncthreads();
    for (int b = tid; b < NB1; b += NT) sm.hist[b] = 0u;
    __syncthreads();
  }
  for (int base = 0; full && base < n; base += kTopkU * NT * 4) {
    if (!(whole_pre && base == 0)) {
#pragma unroll
      for (int u = 0; u < kTopkU; ++u) v[u] = load4(row, base + (u * NT + tid) * 4, n);
    }
#pragma unroll
    for (int u = 0; u < kTopkU; ++u) {
      const int s0 = base + (u * NT + tid) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (s0 + e >= n) continue;
        const uint32_t key = score_key(f4(v[u], e));
        atomicAdd(&sm.hist[key >> (32 - kTopkBits1)], 1u);
        if (whole) {
          sm.ckey[s0 + e] = key;
          sm.cslot[s0 + e] = s0 + e;
        }
      }
    }
  }
  __syncthreads();
  find_bin<NT>(sm.hist, NB1, m, sm.scratch, &sm.sh_bin, &sm.sh_above);
  const uint32_t b1 = sm.sh_bin;
  const uint32_t rem = m - sm.sh_above;
  const uint32_t cand_total = sm.sh_above + sm.hist[b1];
  __syncthreads();  // hist is reused below

  int ncand;
  if (whole) {
    ncand = n;
  } else if (!full && gathered <= (uint32_t)kTopkCap) {
    ncand = (int)gathered;  // every key of bins >= b1 (>= b_est) is staged, in index order
  } else if (cand_total <= (uint32_t)kTopkCap) {
    // ---- pass 2: gather every key with first digit >= b1 into LDS, in index order
    constexpr int E = 4 * kTopkU;
    uint32_t running = 0;
    float4 nx[kTopkU];
#pragma unroll
    for (int u = 0; u < kTopkU; ++u) nx[u] = load4(row, tid * E + 4 * u, n);
    for (int base = 0; base < n; base += E * NT) {
      const int s0 = base + tid * E;
      float4 v[kTopkU];
#pragma unroll
      for (int u = 0; u < kTopkU; ++u) v[u] = nx[u];
      if (base + E * NT < n) {
#pragma unroll
        for (int u = 0; u < kTopkU; ++u) nx[u] = load4(row, s0 + E * NT + 4 * u, n);
      }
      uint32_t key[E];
      uint32_t cnt = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        key[e] = score_key(f4(v[e >> 2], e & 3));
        if (s0 + e < n && (key[e] >> (32 - kTopkBits1)) >= b1) ++cnt;
      }
      uint32_t tot;
      uint32_t p = running + block_exclusive_sum<NT>(cnt, sm.scratch, &tot);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (s0 + e < n && (key[e] >> (32 - kTopkBits1)) >= b1) {
          sm.ckey[p] = key[e];
          sm.cslot[p] = s0 + e;
          ++p;
        }
      }
      running += tot;
    }
    ncand = (int)running;
    __syncthreads();
  } else {
    ncand = -1;  // fall back to passes over the row in memory
  }
  select_finish<NT>(sm, ncand, b1, rem, row, n, m, list, out, outs);
}

// Top-m of short rows (Refine member rows of at most kSmallMax candidates):
// one wave per row (wave_row_select), kSmallWaves rows per workgroup.
__global__ __launch_bounds__(kSmallWaves * kWave) void topk_small_kernel(TopkArgs a) {
  __shared__ uint32_t cand_all[kSmallWaves][kSmallCand];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, so the row's
  const int i = blockIdx.x * kSmallWaves + wid;                       // addresses are scalar
  if (i >= a.nrows) return;
  const int R = a.row_begin + i;
  const float* row = a.S + (long long)i * a.ldS;
  int32_t* out = a.out + (long long)i * a.ldo;
  float* outs = a.out_s ? a.out_s + (long long)i * a.ldos : nullptr;
  const uint32_t m = (uint32_t)a.m;
  const int32_t* list;
  int t;
  refine_row_list(a, R, &list, &t);
  if (!list) {
    for (int s = lane; s < (int)m; s += kWave) {
      out[s] = -1;
      if (outs) outs[s] = no_score();
    }
    return;
  }
  wave_row_select(row, list, a.ldmap, t, m, out, outs, cand_all[wid]);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.nrows <= 0) return hipSuccess;
  // rows whose length is bounded by the candidate list (Refine) fit one wave;
  // with few rows a whole workgroup per row finishes sooner; with at least
  // two rows per compute unit, half-size workgroups let two rows share a
  // compute unit, so one row's barrier waits overlap the other's work
  const bool small = a.kind == kLenRefine && a.ldmap <= kSmallMax && a.nrows >= 1024;
  if (small)
    hipLaunchKernelGGL(topk_small_kernel, dim3((a.nrows + kSmallWaves - 1) / kSmallWaves),
                       dim3(kSmallWaves * kWave), 0, st, a);
  else if (a.nrows >= 512)
    hipLaunchKernelGGL(topk_kernel<kTopkThreadsMany>, dim3(a.nrows), dim3(kTopkThreadsMany), 0, st, a);
  else
    hipLaunchKernelGGL(topk_kernel<kTopkThreads>, dim3(a.nrows), dim3(kTopkThreads), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode top-m: the decode scan has already histogrammed the top 12 key bits
// of every row, so the threshold bin is known up front and a row can be split
// across workgroups.  Gather: each of `parts` workgroups compacts, in index
// order, the keys of its slice whose first digit is at or above the threshold
// bin (the row's first gather workgroup also stores that bin for the
// finalize).  Finalize: one workgroup per row concatenates the slices in LDS
// (they hold at most kTopkCap keys in total) and finishes the radix select; a
// crowded threshold bin (any slice count -1) falls back to passes over the row.
// ---------------------------------------------------------------------------
constexpr int kGatherThreads = 256;

__device__ inline int decode_row_length(const DecSelectArgs& a, int i) {
  if (a.kind == kLenCache) {
    const int nb = a.cache_len[i];
    return (nb < a.g || nb > a.Lmax) ? 0 : max(0, nb - a.excl);
  }
  const int b = i / a.g, nb = a.cache_len[b];
  return (nb < a.g || nb > a.Lmax) ? 0 : max(0, nb - a.g + i % a.g + 1 - a.excl);
}

// Threshold bin of the rem-th largest key from a global 4096-bin histogram,
// NT threads, each owning 4096/NT consecutive bins from the top.
template <int NT>
__device__ inline void find_bin_global(const uint32_t* hist, uint32_t rem, uint32_t* scratch, uint32_t* sh_bin,
                                       uint32_t* sh_above) {
  constexpr int BPT = kSelectBins1 / NT;
  const int tid = threadIdx.x;
  uint32_t c[BPT], sum = 0u;
#pragma unroll
  for (int e = 0; e < BPT; ++e) {
    c[e] = hist[kSelectBins1 - 1 - tid * BPT - e];
    sum += c[e];
  }
  uint32_t tot;
  uint32_t run = block_exclusive_sum<NT>(sum, scratch, &tot);
#pragma unroll
  for (int e = 0; e < BPT; ++e) {
    if (run < rem && rem <= run + c[e]) {
      *sh_bin = (uint32_t)(kSelectBins1 - 1 - tid * BPT - e);
      *sh_above = run;
    }
    run += c[e];
  }
  __syncthreads();
}

__global__ __launch_bounds__(kGatherThreads) void dec_gather_kernel(DecSelectArgs a) {
  constexpr int NT = kGatherThreads;
  constexpr int E = 16;  // elements per thread per round
  __shared__ uint32_t scratch[NT / kWave + 1];
  __shared__ uint32_t sh_bin, sh_above;
  const int i = blockIdx.y, p = blockIdx.x, tid = threadIdx.x;
  const int n = decode_row_length(a, i);
  const uint32_t m = (uint32_t)a.m;
  if (n <= (int)m) return;
  const uint32_t* h = a.hist + (size_t)i * kSelectBins1;
  find_bin_global<NT>(h, m, scratch, &sh_bin, &sh_above);
  const uint32_t b1 = sh_bin;
  const uint32_t cand_total = sh_above + h[b1];
  if (p == 0 && tid == 0) {  // the finalize takes the threshold bin from here
    a.thr[2 * i] = b1;
    a.thr[2 * i + 1] = sh_above;
  }
  int32_t* cnt_out = a.ccount + (size_t)i * a.parts + p;
  if (cand_total > (uint32_t)kTopkCap) {
    if (tid == 0) *cnt_out = -1;
    return;
  }
  const int per = ((n + a.parts - 1) / a.parts + 15) / 16 * 16;
  const int lo = p * per, hi = min(n, lo + per);
  uint32_t* rkey = a.ckey + ((size_t)i * a.parts + p) * a.cap;
  int32_t* rslot = a.cslot + ((size_t)i * a.parts + p) * a.cap;
  const float* row = a.S + (long long)i * a.ldS;
  uint32_t running = 0;
  for (int base = lo; base < hi; base += E * NT) {
    const int s0 = base + tid * E;
    float4 v[E / 4];
#pragma unroll
    for (int u = 0; u < E / 4; ++u) v[u] = load4(row, s0 + 4 * u, hi);
    uint32_t key[E];
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      key[e] = score_key(f4(v[e >> 2], e & 3));
      if (s0 + e < hi && (key[e] >> (32 - kTopkBits1)) >= b1) ++cnt;
    }
    uint32_t tot;
    uint32_t q = running + block_exclusive_sum<NT>(cnt, scratch, &tot);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (s0 + e < hi && (key[e] >> (32 - kTopkBits1)) >= b1) {
        rkey[q] = key[e];
        rslot[q] = s0 + e;
        ++q;
      }
    }
    running += tot;
  }
  if (tid == 0) *cnt_out = (int32_t)running;
}

__global__ __launch_bounds__(kTopkThreads) void dec_finalize_kernel(DecSelectArgs a) {
  constexpr int NT = kTopkThreads;
  __shared__ SelectShared sm;
  __shared__ int sh_bad;
  const int i = blockIdx.x, tid = threadIdx.x;
  // the row length, the threshold bin found by the gather and the slice
  // counts are loaded together
  const int32_t* cnt = a.ccount + (size_t)i * a.parts;
  const int c_own = tid < a.parts ? cnt[tid] : 0;
  const uint32_t b1 = a.thr[2 * i], above = a.thr[2 * i + 1];
  const int n = decode_row_length(a, i);
  const uint32_t m = (uint32_t)a.m;
  const float* row = a.S + (long long)i * a.ldS;
  int32_t* out = a.out + (long long)i * a.ldo;
  float* outs = a.out_s ? a.out_s + (long long)i * a.ldos : nullptr;
  if (n <= (int)m) {
    for (int s = tid; s < (int)m; s += NT) {
      out[s] = s < n ? s : -1;
      if (outs) outs[s] = s < n ? row[s] : no_score();
    }
    return;
  }
  if (tid == 0) sh_bad = 0;
  __syncthreads();
  if (c_own < 0) sh_bad = 1;
  __syncthreads();
  const uint32_t rem = m - above;
  if (sh_bad) {
    select_finish(sm, -1, b1, rem, row, n, m, nullptr, out, outs);
    return;
  }
  // concatenate the slices in order: slice offsets first, then every entry
  // copied in parallel (entry e belongs to the last slice starting at or before e)
  __shared__ int sh_off[kTopkThreads + 1];
  uint32_t tot;
  const uint32_t ex = block_exclusive_sum<NT>((uint32_t)c_own, sm.scratch, &tot);
  if (tid < a.parts) sh_off[tid] = (int)ex;
  if (tid == 0) sh_off[a.parts] = (int)tot;
  __syncthreads();
  const int total = min((int)tot, kTopkCap);
  // entry e (of total <= kTopkCap) comes from the last slice starting at or
  // before e; every load of a thread is issued before its entries are stored
  constexpr int PER = (kTopkCap + NT - 1) / NT;
  uint32_t kk[PER];
  int32_t ss[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + u * NT;
    if (e < total) {
      int lo = 0, hi = a.parts - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sh_off[mid] <= e) lo = mid; else hi = mid - 1;
      }
      const size_t src = ((size_t)i * a.parts + lo) * a.cap + (e - sh_off[lo]);
      kk[u] = a.ckey[src];
      ss[u] = a.cslot[src];
    }
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + u * NT;
    if (e < total) {
      sm.ckey[e] = kk[u];
      sm.cslot[e] = ss[u];
    }
  }
  __syncthreads();
  select_finish(sm, total, b1, rem, row, n, m, nullptr, out, outs);
}

hipError_t launch_decode_select(const DecSelectArgs& a, hipStream_t st) {
  if (a.nrows <= 0) return hipSuccess;
  hipLaunchKernelGGL(dec_gather_kernel, dim3(a.parts, a.nrows), dim3(kGatherThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dec_finalize_kernel, dim3(a.nrows), dim3(kTopkThreads), 0, st, a);
  return hipGetLastError();
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

// Index rows of one layer handed to another (cross-layer reuse): a plain
// copy, 16 bytes per thread and step when both ends allow it.
__global__ void copy_i32_kernel(const int32_t* __restrict__ src, int32_t* __restrict__ dst, size_t n, int vec) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (vec) {
    const size_t n4 = n / 4;
    for (; i < n4; i += stride) reinterpret_cast<i32x4*>(dst)[i] = reinterpret_cast<const i32x4*>(src)[i];
    for (size_t e = n4 * 4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) dst[e] = src[e];
  } else {
    for (; i < n; i += stride) dst[i] = src[i];
  }
}

hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int vec = ((uintptr_t)src % 16 == 0 && (uintptr_t)dst % 16 == 0) ? 1 : 0;
  const size_t units = vec ? (n + 3) / 4 : n;
  const int blocks = (int)std::min<size_t>((units + 255) / 256, 4096);
  hipLaunchKernelGGL(copy_i32_kernel, dim3(blocks), dim3(256), 0, st, src, dst, n, vec);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Reuse (arXiv:2607.24593 abstract: the proxy top-k is shared by the group).
// Member t keeps the entries of the ascending proxy list that are <= t, which
// form a prefix; the rest of its row is -1.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void broadcast_kernel(BroadcastArgs a) {
  const int R = a.row_begin + blockIdx.x;
  int j, t;
  if (a.decode) {
    j = R / a.g;
    const int nb = a.cache_len[j];
    t = (nb < a.g || nb > a.Lmax) ? -1 : nb - a.g + R % a.g - a.excl;
  } else {
    j = R / a.g;
    t = R - a.excl;
  }
  const int32_t* p = a.ptop + (size_t)(j - a.grp_begin) * a.ldp;
  int32_t* out = a.out + (size_t)blockIdx.x * (a.ldo ? a.ldo : a.topk);
  float* outs = a.out_s ? a.out_s + (size_t)blockIdx.x * a.ldos : nullptr;
  const float* srow = a.S ? a.S + (size_t)(j - a.grp_begin) * a.ldS : nullptr;
  for (int s = threadIdx.x; s < a.topk; s += 256) {
    const int v = p[s];
    const bool keep = v >= 0 && v <= t;
    out[s] = keep ? v : -1;
    if (outs) outs[s] = keep ? srow[v] : no_score();
  }
}

hipError_t launch_broadcast(const BroadcastArgs& a, hipStream_t st) {
  const int n = a.row_end - a.row_begin;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(broadcast_kernel, dim3(n), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Sliding window added to the selection (tutorial "Sparse Attention의
// Indexer", section on combining the recent window with the selected
// positions, Figure 3): the window of size W at position t is
// max(0, t-W+1)..t, and each position of the union is read once.  The
// selection is ascending, so its entries below the window form a prefix; the
// row keeps that prefix and continues with the window, in place.  With the
// window excluded from the candidates the selection lies entirely below the
// window and the same step appends it.
// ---------------------------------------------------------------------------
constexpr int kWindowThreads = 256;

__global__ __launch_bounds__(kWindowThreads) void window_union_kernel(WindowArgs a) {
  __shared__ uint32_t scratch[kWindowThreads / kWave + 1];
  const int i = blockIdx.x, tid = threadIdx.x;
  int32_t* row = a.out + (long long)i * a.ldo;
  int t;
  if (a.decode) {
    const int nb = a.cache_len[i / a.g];
    t = (nb < a.g || nb > a.Lmax) ? -1 : nb - a.g + i % a.g;
  } else {
    t = a.row_begin + i;
  }
  const int lo = max(0, t - a.W + 1);
  // entries of the selection below the window (the selection's -1 tail and
  // its entries inside the window are not counted)
  uint32_t c = 0;
  for (int e = tid; e < a.topk; e += kWindowThreads) {
    const int v = row[e];
    c += (v >= 0 && v < lo) ? 1u : 0u;
  }
  uint32_t keep;
  block_exclusive_sum<kWindowThreads>(c, scratch, &keep);  // ends with a barrier: reads done
  const int nwin = t < 0 ? 0 : t - lo + 1;
  for (int e = (int)keep + tid; e < a.topk + a.W; e += kWindowThreads) {
    const int u = e - (int)keep;
    row[e] = u < nwin ? lo + u : -1;
  }
}

hipError_t launch_window_union(const WindowArgs& a, hipStream_t st) {
  if (a.rows <= 0 || a.W <= 0) return hipSuccess;
  hipLaunchKernelGGL(window_union_kernel, dim3(a.rows), dim3(kWindowThreads), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Layout self-test of the 32x32 matrix-core tiles (bf16 and fp8).
// out[(p*2 + f)*1024 + lane*16 + i] for probe p in {row, column, pairing},
// format f in {bf16, fp8}.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void selftest_mfma_kernel(int32_t* out) {
  const int lane = threadIdx.x, hf = lane >> 5, n = lane & 31;
  // bf16: A[i][k0] = i (row probe) / 1 (column probe), B[k0][j] = 1 / j,
  // where k0 is element 0 of lane half 0.
  {
    auto bf = [](float x) { return (short)(__float_as_uint(x) >> 16); };
    typedef short s8 __attribute__((ext_vector_type(8)));
    s8 a{}, b{};
    a[0] = hf == 0 ? bf((float)n) : 0;
    b[0] = hf == 0 ? bf(1.f) : 0;
    f32x16 c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), f32x16{}, 0, 0, 0);
    for (int i = 0; i < 16; ++i) out[0 * 1024 + lane * 16 + i] = (int)c[i];
    a[0] = hf == 0 ? bf(1.f) : 0;
    b[0] = hf == 0 ? bf((float)n) : 0;
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), f32x16{}, 0, 0, 0);
    for (int i = 0; i < 16; ++i) out[2 * 1024 + lane * 16 + i] = (int)c[i];
    // pairing: a one in element 5 of lane half 1 for A and B -> all ones
    s8 a2{}, b2{};
    a2[5] = hf == 1 ? bf(1.f) : 0;
    b2[5] = hf == 1 ? bf(1.f) : 0;
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a2),
                                                __builtin_bit_cast(bf16x8, b2), f32x16{}, 0, 0, 0);
    for (int i = 0; i < 16; ++i) out[4 * 1024 + lane * 16 + i] = (int)c[i];
  }
  // fp8 (E4M3): row i is encoded as 2^(i/8) * (1 + (i%8)/8) = code ((i/8 + 7) << 3) | (i%8),
  // decoded back to i from the float result on the host side of this kernel.
  {
    i32x8 a{}, b{};
    const int code_row = ((n / 8 + 7) << 3) | (n % 8);
    const int one = 0x38;
    a[0] = hf == 0 ? code_row : 0;
    b[0] = hf == 0 ? one : 0;
    f32x16 c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, f32x16{}, 0, 0, 0, 127, 0, 127);
    for (int i = 0; i < 16; ++i) {
      const float v = c[i];
      const int e = ilogbf(v);
      const int m = (int)(ldexpf(v, 3 - e)) - 8;
      out[1 * 1024 + lane * 16 + i] = e * 8 + m;
    }
    a[0] = hf == 0 ? one : 0;
    b[0] = hf == 0 ? code_row : 0;
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, f32x16{}, 0, 0, 0, 127, 0, 127);
    for (int i = 0; i < 16; ++i) {
      const float v = c[i];
      const int e = ilogbf(v);
      const int m = (int)(ldexpf(v, 3 - e)) - 8;
      out[3 * 1024 + lane * 16 + i] = e * 8 + m;
    }
    i32x8 a2{}, b2{};
    a2[6] = hf == 1 ? (one << 16) : 0;  // byte 26 of lane half 1
    b2[6] = hf == 1 ? (one << 16) : 0;
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a2, b2, f32x16{}, 0, 0, 0, 127, 0, 127);
    for (int i = 0; i < 16; ++i) out[5 * 1024 + lane * 16 + i] = (int)c[i];
  }
}

hipError_t launch_selftest_mfma(int32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(selftest_mfma_kernel, dim3(1), dim3(64), 0, st, out);
  return hipGetLastError();
}

}  // namespace pivot
