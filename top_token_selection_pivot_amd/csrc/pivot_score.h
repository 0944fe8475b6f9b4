// pivot_score.h -- indexer scoring kernels (gfx950).
//
// Score of query row r against key s (arXiv:2607.24593's DSA indexer with the
// weighted-ReLU multi-head score; tutorial "Sparse Attention의 Indexer",
// Figure 1, for the single-head dot product):
//     S[r][s] = sum_h w[r][h] * max(0, q[r][h] . k[s])      (bf16)
//     S[r][s] = s_q[r] * s_k[s] * sum_h w[r][h] * max(0, q[r][h] . k[s])   (fp8 codes)
// computed as a matrix-core contraction over D with the heads on the M axis,
// fused with the ReLU, the head weights and the head sum; only the final
// per-(row, key) score is written.
//
// Three kernels:
//  * scan_kernel:        8 query rows per workgroup (one wave each) share
//                        32-key tiles staged in LDS; causal: row r stops at pos(r).
//  * refine_kernel:      the members of one group score the group's candidate
//                        keys, gathered from the key cache into LDS.
//  * decode_scan_kernel: one sequence's 1-2 query rows stream that sequence's
//                        key cache straight into registers (no reuse to stage).
#pragma once

#include "pivot_device.h"
#include "pivot_kernels.h"

namespace pivot {

constexpr int kScanRows = 8;      // query rows (waves) per scan workgroup
constexpr int kScanThreads = kScanRows * kWave;
constexpr int kLdsPad = 16;       // bytes of padding per staged key row

// Per-wave query state: A fragments of every head block and contraction step,
// and the head weight of every accumulator this lane holds.
template <int DT, int D, int HB>
struct QueryRegs {
  static constexpr int NKS = D / Fmt<DT>::KSTEP;
  typename Fmt<DT>::frag a[HB][NKS];
  float wv[HB][16];

  __device__ inline void load(const uint8_t* qrow, const float* wrow, int H, int lane) {
    const int hf = lane >> 5;
#pragma unroll
    for (int mb = 0; mb < HB; ++mb) {
      const int h = mb * 32 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        a[mb][ks] = h < H ? load_frag<DT>(qrow + (size_t)h * D * Fmt<DT>::ESZ +
                                          frag_offset<DT, D>(ks, hf))
                          : zero_frag<DT>();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hh = mb * 32 + acc_row(i, lane);
        wv[mb][i] = hh < H ? wrow[hh] : 0.0f;
      }
    }
  }
};

// Contract one 32-key tile whose B fragments are produced by `bfrag(ks)`, then
// apply ReLU, head weights and the head sum.  Returns, in lanes 0..31, the
// score of key (tile + lane) (lanes 32..63 hold the same values).
template <int DT, int D, int HB, typename BF>
__device__ inline float score_tile(const QueryRegs<DT, D, HB>& qr, BF bfrag) {
  constexpr int NKS = D / Fmt<DT>::KSTEP;
  f32x16 acc[HB];
#pragma unroll
  for (int mb = 0; mb < HB; ++mb) acc[mb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const typename Fmt<DT>::frag b = bfrag(ks);
#pragma unroll
    for (int mb = 0; mb < HB; ++mb) acc[mb] = Fmt<DT>::mma(qr.a[mb][ks], b, acc[mb]);
  }
  float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
  for (int mb = 0; mb < HB; ++mb) {
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      p0 = fmaf(qr.wv[mb][i + 0], fmaxf(acc[mb][i + 0], 0.f), p0);
      p1 = fmaf(qr.wv[mb][i + 1], fmaxf(acc[mb][i + 1], 0.f), p1);
      p2 = fmaf(qr.wv[mb][i + 2], fmaxf(acc[mb][i + 2], 0.f), p2);
      p3 = fmaf(qr.wv[mb][i + 3], fmaxf(acc[mb][i + 3], 0.f), p3);
    }
  }
  float part = (p0 + p1) + (p2 + p3);
  return part + __shfl_xor(part, 32, 64);
}

// Staged key tile in LDS: kTileN rows of D codes, padded.
template <int DT, int D>
struct KeyTile {
  static constexpr int ROW = D * Fmt<DT>::ESZ;       // bytes of one key row
  static constexpr int STRIDE = ROW + kLdsPad;
  static constexpr int CHUNKS = kTileN * ROW / 16;   // 16-byte pieces per tile
  static constexpr int BYTES = kTileN * STRIDE;
};

// ---------------------------------------------------------------------------
// Prefill full-prefix scan.
// ---------------------------------------------------------------------------
template <int DT, int D, int HB>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(ScanArgs a) {
  using KT = KeyTile<DT, D>;
  constexpr int NPT = (KT::CHUNKS + kScanThreads - 1) / kScanThreads;
  __shared__ __attribute__((aligned(16))) uint8_t tile[KT::BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int rb = a.row_begin + blockIdx.y * kScanRows;
  const int rlast = min(rb + kScanRows, a.row_end) - 1;
  const int lim = min(rlast * a.pos_mul + a.pos_add, a.pos_cap) + 1;  // keys 0..lim-1
  const int k0 = blockIdx.x * a.kc;
  if (k0 >= lim) return;
  const int k1 = min(k0 + a.kc, lim);

  const int r = rb + wid;
  const bool active = r <= rlast;
  const int pos = active ? min(r * a.pos_mul + a.pos_add, a.pos_cap) : -1;

  QueryRegs<DT, D, HB> qr;
  float qs = 1.f;
  if (active) {
    qr.load(a.q + (size_t)r * a.H * D * Fmt<DT>::ESZ, a.w + (size_t)r * a.H, a.H, lane);
    if constexpr (DT == kFP8) qs = a.q_scale[r];
  }

  i32x4 pre[NPT];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int c = tid + i * kScanThreads;
      pre[i] = i32x4{};
      if (c < KT::CHUNKS) {
        const int key = t0 + c / (KT::ROW / 16);
        if (key < a.Lk)
          pre[i] = *reinterpret_cast<const i32x4*>(a.k + (size_t)key * KT::ROW +
                                                   (c % (KT::ROW / 16)) * 16);
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int c = tid + i * kScanThreads;
      if (c < KT::CHUNKS)
        *reinterpret_cast<i32x4*>(tile + (c / (KT::ROW / 16)) * KT::STRIDE +
                                  (c % (KT::ROW / 16)) * 16) = pre[i];
    }
  };

  float* srow = a.S + (long long)(r - a.row_begin) * a.ldS;
  const int hf = lane >> 5, n = lane & 31;
  fetch(k0);
  for (int t0 = k0; t0 < k1; t0 += kTileN) {
    __syncthreads();
    stash();
    __syncthreads();
    if (t0 + kTileN < k1) fetch(t0 + kTileN);
    if (active && t0 <= pos) {
      const uint8_t* brow = tile + n * KT::STRIDE;
      float s = score_tile<DT, D, HB>(qr, [&](int ks) {
        return load_frag<DT>(brow + frag_offset<DT, D>(ks, hf));
      });
      const int key = t0 + lane;
      if (lane < kTileN && key <= pos && key < k1) {
        if constexpr (DT == kFP8) s = (s * qs) * a.k_scale[key];
        srow[key] = s;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Refine: members of one group score the group's candidates.
// ---------------------------------------------------------------------------
template <int DT, int D, int HB>
__global__ __launch_bounds__(kScanThreads) void refine_kernel(RefineArgs a) {
  using KT = KeyTile<DT, D>;
  __shared__ __attribute__((aligned(16))) uint8_t tile[KT::BYTES];
  __shared__ int32_t tpos[kTileN];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nthreads = blockDim.x;
  const int j = a.grp_begin + blockIdx.y;

  // group geometry
  int row0, nmem, ncand;
  size_t keybase = 0;
  const float* kscale = a.k_scale;
  if (a.kind == 0) {
    row0 = j * a.g;
    nmem = min(a.g, a.L - row0);
    ncand = min(a.m, row0 + nmem);  // min(m, e_j + 1)
  } else {
    const int nb = a.cache_len[j];
    if (nb < a.g || nb > a.Lmax) return;
    row0 = j * a.g;
    nmem = a.g;
    ncand = min(a.m, nb);
    keybase = (size_t)j * a.Lmax;
    if constexpr (DT == kFP8) kscale += keybase;
  }
  const int s0 = blockIdx.x * a.slot_chunk;
  if (s0 >= ncand) return;
  const int s1 = min(s0 + a.slot_chunk, ncand);
  const int mem = blockIdx.z * kScanRows + wid;
  const bool active = mem < nmem;
  const int r = row0 + mem;
  const int32_t* cand = a.cand + (size_t)(j - a.grp_begin) * a.ldc;
  const uint8_t* kb = a.k + keybase * KT::ROW;

  QueryRegs<DT, D, HB> qr;
  float qs = 1.f;
  if (active) {
    qr.load(a.q + (size_t)r * a.H * D * Fmt<DT>::ESZ, a.w + (size_t)r * a.H, a.H, lane);
    if constexpr (DT == kFP8) qs = a.q_scale[r];
  }
  float* srow = a.S + (long long)(r - a.row_base) * a.ldS;
  const int hf = lane >> 5, n = lane & 31;

  for (int t0 = s0; t0 < s1; t0 += kTileN) {
    __syncthreads();
    if (tid < kTileN) tpos[tid] = (t0 + tid < s1) ? cand[t0 + tid] : -1;
    __syncthreads();
    for (int c = tid; c < KT::CHUNKS; c += nthreads) {
      const int kr = c / (KT::ROW / 16), part = c % (KT::ROW / 16);
      const int p = tpos[kr];
      i32x4 v = i32x4{};
      if (p >= 0) v = *reinterpret_cast<const i32x4*>(kb + (size_t)p * KT::ROW + part * 16);
      *reinterpret_cast<i32x4*>(tile + kr * KT::STRIDE + part * 16) = v;
    }
    __syncthreads();
    if (active) {
      const uint8_t* brow = tile + n * KT::STRIDE;
      float s = score_tile<DT, D, HB>(qr, [&](int ks) {
        return load_frag<DT>(brow + frag_offset<DT, D>(ks, hf));
      });
      const int slot = t0 + lane;
      if (lane < kTileN && slot < s1) {
        if constexpr (DT == kFP8) s = (s * qs) * kscale[tpos[lane]];
        srow[slot] = s;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode scan: QR query rows of one sequence stream its key cache.
// ---------------------------------------------------------------------------
constexpr int kDecThreads = 256;

template <int DT, int D, int HB, int QR>
__global__ __launch_bounds__(kDecThreads) void decode_scan_kernel(DecScanArgs a) {
  constexpr int NKS = D / Fmt<DT>::KSTEP;
  constexpr int ROW = D * Fmt<DT>::ESZ;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.y;
  const int nb = a.cache_len[b];
  if (nb < a.g || nb > a.Lmax) return;
  const int k0 = blockIdx.x * a.kc;
  if (k0 >= nb) return;
  const int k1 = min(k0 + a.kc, nb);

  // rows of this workgroup: qr rows per sequence, QR at a time (blockIdx.z)
  const int ri0 = blockIdx.z * QR;
  QueryRegs<DT, D, HB> q[QR];
  float qs[QR];
  int pos[QR];
#pragma unroll
  for (int i = 0; i < QR; ++i) {
    const int ri = ri0 + i;
    pos[i] = -1;
    qs[i] = 1.f;
    if (ri < a.qr) {
      const size_t row = (size_t)b * a.qr + ri;
      q[i].load(a.q + row * a.H * ROW, a.w + row * a.H, a.H, lane);
      if constexpr (DT == kFP8) qs[i] = a.q_scale[row];
      pos[i] = a.qr == 1 ? nb - 1 : nb - a.g + ri;
    }
  }
  const uint8_t* kb = a.k + (size_t)b * a.Lmax * ROW;
  const float* ksc = a.k_scale + (DT == kFP8 ? (size_t)b * a.Lmax : 0);
  const int hf = lane >> 5, n = lane & 31;

  for (int t0 = k0 + wid * kTileN; t0 < k1; t0 += (kDecThreads / kWave) * kTileN) {
    const int key = min(t0 + n, k1 - 1);
    typename Fmt<DT>::frag bf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      bf[ks] = load_frag<DT>(kb + (size_t)key * ROW + frag_offset<DT, D>(ks, hf));
    float ksv = 1.f;
    if constexpr (DT == kFP8) ksv = ksc[min(t0 + lane, k1 - 1)];
#pragma unroll
    for (int i = 0; i < QR; ++i) {
      if (pos[i] < 0 || t0 > pos[i]) continue;
      float s = score_tile<DT, D, HB>(q[i], [&](int ks) { return bf[ks]; });
      const int kk = t0 + lane;
      if (lane < kTileN && kk <= pos[i] && kk < k1) {
        if constexpr (DT == kFP8) s = (s * qs[i]) * ksv;
        a.S[((size_t)b * a.qr + ri0 + i) * a.ldS + kk] = s;
      }
    }
  }
}

}  // namespace pivot
