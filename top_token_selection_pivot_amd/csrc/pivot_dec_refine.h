// pivot_dec_refine.h -- decode PIVOT-Refine fused with the member top-k.
//
// In a decode step every member of a group (the queries of one multi-token
// prediction step, arXiv:2607.24593 abstract) re-scores the proxy's candidates
// with its own query and keeps its own causal top-k.  With only B*g member
// rows the separate score and select launches are latency-bound, so one
// workgroup takes one member row end to end:
//   1. the candidate list is read once: the gather row of every slot goes to
//      LDS and the slots <= the member's limit are counted (a prefix, since
//      the list is ascending);
//   2. each wave scores 32-key tiles of those slots on the matrix cores
//      (heads on M, the gathered keys on N, the member's query in registers),
//      loading the B fragments of a batch of tiles straight from the cache
//      before contracting any of them, and stores the scores' order-preserving
//      keys in LDS;
//   3. the exact top-k of the LDS row: a 12-bit first digit, then the shared
//      selection finish (two 10-bit digits, index-ordered emission, ties to
//      the lower position).
#pragma once

#include "pivot_score.h"
#include "pivot_select.h"

namespace pivot {

constexpr int kDecRefThreads = 512;
constexpr int kDecRefWaves = kDecRefThreads / kWave;

// tiles whose key fragments a wave keeps in flight: what is left of 256
// registers after the query fragments (two head blocks), the 32 head weights,
// one tile's accumulators and about 24 for the rest
template <int DT, int D>
constexpr int dec_ref_batch() {
  constexpr int per_tile = D * Fmt<DT>::ESZ / 2 / 4;  // half a key row per lane
  constexpr int query = 2 * per_tile;
  constexpr int avail = 256 - 24 - 32 - 32 - query;
  return avail >= 8 * per_tile ? 8 : avail >= 4 * per_tile ? 4 : avail >= 2 * per_tile ? 2 : 1;
}

// shapes whose query fragments leave room for a batch of key fragments
template <int DT, int D>
constexpr bool dec_ref_fits() {
  return D * Fmt<DT>::ESZ <= 256;
}
inline bool dec_ref_fits_rt(int dtype, int D) { return D * (dtype == kBF16 ? 2 : 1) <= 256; }

template <int DT, int D, int HB>
__global__ __launch_bounds__(kDecRefThreads) void dec_refine_select_kernel(DecRefineArgs a) {
  using Frag = typename Fmt<DT>::frag;
  constexpr int NT = kDecRefThreads;
  constexpr int NKS = D / Fmt<DT>::KSTEP;
  constexpr int ROW = D * Fmt<DT>::ESZ;
  constexpr int TB = dec_ref_batch<DT, D>();
  __shared__ SelectShared sm;
  __shared__ int32_t crow[kRefineSlotMax];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = blockIdx.x;
  const int b = r / a.g, mi = r % a.g;
  const int nb = a.cache_len[b];
  int32_t* out = a.out + (long long)r * a.ldo;
  float* outs = a.out_s ? a.out_s + (long long)r * a.ldos : nullptr;
  const int m = a.topk;
  if (nb < a.g || nb > a.Lmax) {
    for (int s = tid; s < m; s += NT) {
      out[s] = -1;
      if (outs) outs[s] = no_score();
    }
    return;
  }
  const int t = nb - a.g + mi - a.excl;  // the member's last selectable position
  const int ncand = min(a.m, max(0, nb - a.excl));
  const int32_t* list = a.cand + (size_t)b * a.ldc;

  // 1. gather rows of the slots, and the member's pool size n
  uint32_t cnt = 0;
  for (int s = tid; s < ncand; s += NT) {
    const int v = list[s];
    cnt += (v >= 0 && v <= t) ? 1u : 0u;
    int row = max(v, 0);
    if (a.bt) {
      const int pg = a.bt[(size_t)b * a.bt_stride + (row >> a.page_shift)];
      row = (unsigned)pg < (unsigned)(a.pool_rows >> a.page_shift)
                ? (pg << a.page_shift) + (row & ((1 << a.page_shift) - 1))
                : a.pool_rows;  // past the pool: reads as zeros
    }
    crow[s] = row;
  }
  uint32_t n_u;
  block_exclusive_sum<NT>(cnt, sm.scratch, &n_u);  // its barriers also publish crow
  const int n = (int)n_u;

  // 2. scores of slots [0, n) as keys in sm.ckey (slot order)
  const uint8_t* kbase = a.bt ? a.k : a.k + (size_t)b * a.Lmax * ROW;
  const uint32_t nrows = a.bt ? (uint32_t)a.pool_rows : (uint32_t)nb;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, nrows * (uint32_t)ROW);
  const float* sbase = DT == kFP8 ? (a.bt ? a.k_scale : a.k_scale + (size_t)b * a.Lmax) : a.w;
  const __amdgpu_buffer_rsrc_t ksr = make_rsrc(sbase, DT == kFP8 ? nrows * 4u : 0u);
  QueryRegs<DT, D, HB> qr;
  qr.load(a.q + (size_t)r * a.H * ROW, a.w + (size_t)r * a.H, a.H, lane);
  const float qs = DT == kFP8 ? a.q_scale[r] : 1.f;
  const int hf = lane >> 5, nn = lane & 31;
  const int ntiles = (n + kTileN - 1) / kTileN;
  for (int k0 = wid; k0 < ntiles; k0 += kDecRefWaves * TB) {
    Frag bf[TB][NKS];
    float ksv[TB];
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int slot = (k0 + u * kDecRefWaves) * kTileN + nn;
      // slots past the pool read past the buffer: zeros
      const uint32_t base = slot < n ? (uint32_t)crow[slot] * (uint32_t)ROW : 0xFFFFFF00u;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint32_t off = base + (uint32_t)frag_offset<DT, D>(ks, hf);
        if constexpr (DT == kBF16) {
          bf[u][ks] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
        } else {
          const i32x4 lo = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
          const i32x4 hi = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off + 16, 0, 0));
          bf[u][ks] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
      ksv[u] = 1.f;
      if constexpr (DT == kFP8)
        ksv[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            ksr, slot < n ? (uint32_t)crow[slot] * 4u : 0xFFFFFF00u, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int tile = k0 + u * kDecRefWaves;
      if (tile >= ntiles) break;
      float sc = score_tile<DT, D, HB>(qr, [&](int ks) { return bf[u][ks]; });
      if constexpr (DT == kFP8) sc = (sc * qs) * ksv[u];
      const int slot = tile * kTileN + nn;
      if (hf == 0 && slot < n) {
        sm.ckey[slot] = score_key(sc);
        sm.cslot[slot] = slot;
      }
    }
  }
  __syncthreads();

  // 3. the member's top-k of the n scored slots
  if (n <= m) {
    for (int s = tid; s < m; s += NT) {
      out[s] = s < n ? list[s] : -1;
      if (outs) outs[s] = s < n ? key_score(sm.ckey[s]) : no_score();
    }
    return;
  }
  constexpr int NB1 = kSelectBins1;
  for (int e = tid; e < NB1; e += NT) sm.hist[e] = 0u;
  __syncthreads();
  for (int s = tid; s < n; s += NT) atomicAdd(&sm.hist[sm.ckey[s] >> 20], 1u);
  __syncthreads();
  find_bin<NT>(sm.hist, NB1, (uint32_t)m, sm.scratch, &sm.sh_bin, &sm.sh_above);
  const uint32_t b1 = sm.sh_bin;
  const uint32_t rem = (uint32_t)m - sm.sh_above;
  __syncthreads();  // hist is reused below
  select_finish<NT>(sm, n, b1, rem, nullptr, n, (uint32_t)m, list, out, outs);
}

}  // namespace pivot
