// pivot_select.hip -- proxy mean, top-m selection, Reuse broadcast and the
// matrix-core layout self-test (gfx950).
#include "pivot_device.h"
#include "pivot_kernels.h"

namespace pivot {

hipError_t launch_scan_bf16(const ScanArgs&, int, hipStream_t);
hipError_t launch_scan_fp8(const ScanArgs&, int, hipStream_t);
hipError_t launch_refine_bf16(const RefineArgs&, int, hipStream_t);
hipError_t launch_refine_fp8(const RefineArgs&, int, hipStream_t);
hipError_t launch_decode_scan_bf16(const DecScanArgs&, int, int, hipStream_t);
hipError_t launch_decode_scan_fp8(const DecScanArgs&, int, int, hipStream_t);

hipError_t launch_scan(const ScanArgs& a, int dtype, int D, hipStream_t st) {
  return dtype == kBF16 ? launch_scan_bf16(a, D, st) : launch_scan_fp8(a, D, st);
}
hipError_t launch_refine(const RefineArgs& a, int dtype, int D, hipStream_t st) {
  return dtype == kBF16 ? launch_refine_bf16(a, D, st) : launch_refine_fp8(a, D, st);
}
hipError_t launch_decode_scan(const DecScanArgs& a, int dtype, int D, int B, hipStream_t st) {
  return dtype == kBF16 ? launch_decode_scan_bf16(a, D, B, st)
                        : launch_decode_scan_fp8(a, D, B, st);
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
constexpr int kProxyThreads = 256;

template <int DT>
__device__ inline float member_value(const ProxyArgs& a, int row, size_t e) {
  if constexpr (DT == kBF16) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[(size_t)row * a.H * a.D + e]);
  } else {
    return __fmul_rn(a.q_scale[row], e4m3_to_f32(a.q[(size_t)row * a.H * a.D + e]));
  }
}

template <int DT>
__device__ inline float group_mean(const ProxyArgs& a, int r0, int n, size_t e) {
  float s = 0.f;
  for (int t = 0; t < n; ++t) s = __fadd_rn(s, member_value<DT>(a, r0 + t, e));
  return __fdiv_rn(s, (float)n);
}

template <int DT>
__global__ __launch_bounds__(kProxyThreads) void proxy_mean_kernel(ProxyArgs a) {
  const int j = blockIdx.x, tid = threadIdx.x;
  const int r0 = j * a.g;
  const int n = min(a.g, a.R - r0);
  const size_t HD = (size_t)a.H * a.D;
  if (n == 1) {  // a one-member group is its member
    const size_t esz = DT == kBF16 ? 2 : 1;
    for (size_t e = tid; e < HD * esz; e += kProxyThreads)
      a.qbar[j * HD * esz + e] = a.q[(size_t)r0 * HD * esz + e];
    if (tid == 0) a.qbar_scale[j] = DT == kBF16 ? 1.f : a.q_scale[r0];
    for (int h = tid; h < a.H; h += kProxyThreads) a.wbar[(size_t)j * a.H + h] = a.w[(size_t)r0 * a.H + h];
    return;
  }
  for (int h = tid; h < a.H; h += kProxyThreads) {
    float s = 0.f;
    for (int t = 0; t < n; ++t) s = __fadd_rn(s, a.w[(size_t)(r0 + t) * a.H + h]);
    a.wbar[(size_t)j * a.H + h] = __fdiv_rn(s, (float)n);
  }
  if constexpr (DT == kBF16) {
    uint16_t* out = reinterpret_cast<uint16_t*>(a.qbar) + (size_t)j * HD;
    for (size_t e = tid; e < HD; e += kProxyThreads) out[e] = f32_to_bf16_rne(group_mean<DT>(a, r0, n, e));
    if (tid == 0) a.qbar_scale[j] = 1.f;
  } else {
    __shared__ float red[kProxyThreads / kWave];
    float amax = 0.f;
    for (size_t e = tid; e < HD; e += kProxyThreads) amax = fmaxf(amax, fabsf(group_mean<DT>(a, r0, n, e)));
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = red[0];
    for (int i = 1; i < kProxyThreads / kWave; ++i) amax = fmaxf(amax, red[i]);
    const float sp = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
    for (size_t e = tid; e < HD; e += kProxyThreads)
      a.qbar[(size_t)j * HD + e] = f32_to_e4m3_rne_sat(__fdiv_rn(group_mean<DT>(a, r0, n, e), sp));
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

// ---------------------------------------------------------------------------
// Exact top-m of one score row (tutorial "Sparse Attention의 Indexer",
// Figure 1: keep the positions of the m largest scores).  Radix select over
// the order-preserving 32-bit keys, most significant digit first (11, 11 and
// 10 bits, LDS histograms), finds the m-th largest key T and how many keys
// equal to T are taken; an index-ordered compaction then emits every key
// above T and the first such keys equal to T, so equal scores go to the lower
// position and the output is ascending.
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 1024;

__device__ inline int ref_count(const int32_t* list, int m, int t) {
  // number of leading entries of the ascending, -1 padded list that are in [0, t]
  int lo = 0, hi = m;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const int v = list[mid];
    if (v >= 0 && v <= t)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

__device__ inline int row_length(const TopkArgs& a, int R, const int32_t** list) {
  *list = nullptr;
  switch (a.kind) {
    case kLenPos:
      return min(R * a.pos_mul + a.pos_add, a.pos_cap) + 1;
    case kLenCache: {
      const int nb = a.cache_len[R];
      return (nb < a.g || nb > a.Lmax) ? 0 : nb;
    }
    case kLenDecodeDense: {
      const int b = R / a.g, i = R % a.g, nb = a.cache_len[b];
      return (nb < a.g || nb > a.Lmax) ? 0 : nb - a.g + i + 1;
    }
    default: {  // kLenRefine
      int j, t;
      if (a.decode) {
        j = R / a.g;
        const int nb = a.cache_len[j];
        if (nb < a.g || nb > a.Lmax) return 0;
        t = nb - a.g + R % a.g;
      } else {
        j = R / a.g;
        t = R;
      }
      *list = a.map + (size_t)(j - a.map_grp_begin) * a.ldmap;
      return ref_count(*list, a.ldmap, t);
    }
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t scratch[kTopkThreads / kWave + 1];
  __shared__ uint32_t sh_digit, sh_rem;

  const int tid = threadIdx.x;
  const int i = blockIdx.x;
  const int R = a.row_begin + i;
  const float* row = a.S + (long long)i * a.ldS;
  int32_t* out = a.out + (long long)i * a.ldo;
  const int32_t* list;
  const int n = row_length(a, R, &list);
  const int m = a.m;

  if (n <= m) {
    for (int s = tid; s < m; s += kTopkThreads) out[s] = s < n ? (list ? list[s] : s) : -1;
    return;
  }

  uint32_t prefix = 0, pmask = 0, rem = (uint32_t)m;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const uint32_t nb = 1u << widths[pass];
    for (uint32_t b = tid; b < nb; b += kTopkThreads) hist[b] = 0;
    __syncthreads();
    for (int s = tid; s < n; s += kTopkThreads) {
      const uint32_t key = score_key(row[s]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    // thread t owns bins nb-1-2t and nb-2-2t (descending), so an inclusive
    // scan over threads counts keys from the top bin down
    const int b0 = (int)nb - 1 - 2 * tid, b1 = b0 - 1;
    const bool own = 2 * tid < (int)nb;
    const uint32_t c0 = own ? hist[b0] : 0u, c1 = own ? hist[b1] : 0u;
    uint32_t tot;
    const uint32_t excl = block_exclusive_sum<kTopkThreads>(c0 + c1, scratch, &tot);
    if (own) {
      if (excl < rem && rem <= excl + c0) {
        sh_digit = (uint32_t)b0;
        sh_rem = rem - excl;
      } else if (excl + c0 < rem && rem <= excl + c0 + c1) {
        sh_digit = (uint32_t)b1;
        sh_rem = rem - excl - c0;
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    pmask |= (nb - 1) << shift;
    rem = sh_rem;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t need_eq = rem;           // keys equal to T to take, lowest positions first
  const uint32_t need_gt = (uint32_t)m - need_eq;

  uint32_t g_gt = 0, g_eq = 0;
  for (int base = 0; base < n; base += 4 * kTopkThreads) {
    const int s0 = base + 4 * tid;
    uint32_t key[4];
    uint32_t cgt = 0, ceq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      key[e] = s0 + e < n ? score_key(row[s0 + e]) : 0u;
      const bool valid = s0 + e < n;
      cgt += (valid && key[e] > T) ? 1u : 0u;
      ceq += (valid && key[e] == T) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t excl = block_exclusive_sum<kTopkThreads>(cgt | (ceq << 16), scratch, &tot);
    uint32_t gt_before = g_gt + (excl & 0xFFFFu), eq_before = g_eq + (excl >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (s0 + e >= n) break;
      const int slot = s0 + e;
      if (key[e] > T) {
        const uint32_t pos = gt_before + min(eq_before, need_eq);
        if (pos < (uint32_t)m) out[pos] = list ? list[slot] : slot;
        ++gt_before;
      } else if (key[e] == T) {
        const uint32_t pos = gt_before + eq_before;
        if (eq_before < need_eq && pos < (uint32_t)m) out[pos] = list ? list[slot] : slot;
        ++eq_before;
      }
    }
    g_gt += tot & 0xFFFFu;
    g_eq += tot >> 16;
    if (g_gt >= need_gt && g_eq >= need_eq) break;
  }
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.nrows <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(a.nrows), dim3(kTopkThreads), 0, st, a);
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
    t = (nb < a.g || nb > a.Lmax) ? -1 : nb - a.g + R % a.g;
  } else {
    j = R / a.g;
    t = R;
  }
  const int32_t* p = a.ptop + (size_t)(j - a.grp_begin) * a.ldp;
  int32_t* out = a.out + (size_t)blockIdx.x * a.topk;
  for (int s = threadIdx.x; s < a.topk; s += 256) {
    const int v = p[s];
    out[s] = (v >= 0 && v <= t) ? v : -1;
  }
}

hipError_t launch_broadcast(const BroadcastArgs& a, hipStream_t st) {
  const int n = a.row_end - a.row_begin;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(broadcast_kernel, dim3(n), dim3(256), 0, st, a);
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
