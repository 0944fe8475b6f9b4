// pivot_select.h -- the exact top-m selection building blocks of the
// selection kernels (pivot_select.hip): radix digits over order-preserving
// keys in LDS, the threshold-bin search, the index-ordered emission and the
// one-wave selection of short rows.
#pragma once

#include "pivot_device.h"
#include "pivot_kernels.h"

namespace pivot {

// ---------------------------------------------------------------------------
// Exact top-m of one score row (tutorial "Sparse Attention의 Indexer",
// Figure 1: keep the positions of the m largest scores).
//
// Radix select over order-preserving 32-bit keys, most significant digit
// first, with LDS histograms.  It finds the m-th largest key T and how many
// keys equal to T are taken; an index-ordered compaction then emits every key
// above T and the first keys equal to T, so equal scores go to the lower
// position and the output is ascending.
//
// Pass 1 reads the row once (16-byte loads, four in flight per thread) and
// histograms its top 12 bits.  Every key at or above the threshold bin is then
// gathered into LDS in index order (a row that fits is staged whole during
// pass 1); the remaining 20 bits and the emission run on that LDS copy, so a
// row is read from memory at most twice.  A long row is read about once: a
// sixteenth of it is sampled first, and pass 1 gathers the keys at or above a
// conservative bin estimated from the sample while it histograms (pass 2 is
// needed only when the estimate turns out too high or too low).  If the
// threshold bin is too crowded for LDS (e.g. a huge run of equal scores), the
// selection falls back to further passes over the row in memory.
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 1024;     // threads of a one-row workgroup (few rows)
constexpr int kTopkThreadsMany = 512;  // with many rows: two workgroups share a compute unit
constexpr int kTopkCap = kSelectCap;  // keys staged in LDS
constexpr int kTopkBits1 = 12;        // first digit: bits 31..20
static_assert((1 << kTopkBits1) == kSelectBins1, "first-digit histogram width");
constexpr int kTopkU = 4;          // 16-byte loads in flight per thread
constexpr int kTopkSampleMin = 4 * kTopkCap;  // rows this long are sampled first

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
      return (nb < a.g || nb > a.Lmax) ? 0 : max(0, nb - a.excl);
    }
    case kLenDecodeDense: {
      const int b = R / a.g, i = R % a.g, nb = a.cache_len[b];
      return (nb < a.g || nb > a.Lmax) ? 0 : max(0, nb - a.g + i + 1 - a.excl);
    }
    default: {  // kLenRefine
      int j, t;
      if (a.decode) {
        j = R / a.g;
        const int nb = a.cache_len[j];
        if (nb < a.g || nb > a.Lmax) return 0;
        t = nb - a.g + R % a.g - a.excl;
      } else {
        j = R / a.g;
        t = R - a.excl;
      }
      *list = a.map + (size_t)(j - a.map_grp_begin) * a.ldmap;
      return ref_count(*list, a.ldmap, t);
    }
  }
}

// Refine row R: its group's candidate list and the member's position t;
// returns 0 (and no list) for a decode sequence with an invalid length.
__device__ inline int refine_row_list(const TopkArgs& a, int R, const int32_t** list, int* t) {
  const int j = R / a.g;
  *list = nullptr;
  if (a.decode) {
    const int nb = a.cache_len[j];
    if (nb < a.g || nb > a.Lmax) return 0;
    *t = nb - a.g + R % a.g - a.excl;
  } else {
    *t = R - a.excl;
  }
  *list = a.map + (size_t)(j - a.map_grp_begin) * a.ldmap;
  return 0;
}

// The bin (of nbins, a multiple of 256, counted from the top) that holds the
// rem-th largest key; *above receives the number of keys in higher bins.
// One wave walks the histogram in rounds of 256 bins from the top (lane l
// reads the four bins 4l..4l+3 below the round's top with one 16-byte read),
// so the other waves only wait at the closing barrier.
template <int NT>
__device__ inline void find_bin(const uint32_t* hist, int nbins, uint32_t rem, uint32_t* scratch,
                                uint32_t* sh_bin, uint32_t* sh_above) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    uint32_t above = 0;
    for (int k = 0; k < nbins / 256; ++k) {
      const int top = nbins - 1 - (256 * k + 4 * lane);  // the lane's highest bin
      const uint4 v = *reinterpret_cast<const uint4*>(&hist[top - 3]);
      const uint32_t s = v.x + v.y + v.z + v.w;
      const uint32_t inc = wave_inclusive_sum(s);
      const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)inc, kWave - 1);
      if (above + tot >= rem) {
        uint32_t run = above + inc - s;
        const uint32_t c[4] = {v.w, v.z, v.y, v.x};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (run < rem && rem <= run + c[e]) {
            *sh_bin = (uint32_t)(top - e);
            *sh_above = run;
          }
          run += c[e];
        }
        break;
      }
      above += tot;
    }
  }
  __syncthreads();
}

// Loads the 4 scores at s0..s0+3 of a row of n (s0 a multiple of 4), zeros at
// and past n.  One range-checked 16-byte buffer load: the hardware checks each
// dword of it against the range (a load straddling the end returns the dwords
// before it and zeros after), so no branch, and several such loads stay in
// flight together.  `row` must be wave-uniform (a scalar descriptor).
__device__ inline float4 load4(const float* row, int s0, int n) {
  return __builtin_bit_cast(
      float4, __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(row, (uint32_t)n * 4u), s0 * 4, 0, 0));
}

__device__ inline float f4(const float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

// Emits, in index order, the entries of a sequence that are selected by
// (T, need_eq): keys above T, and the first need_eq keys equal to T.  The
// sequence is given by get(i) -> (key, slot) for i < cnt; each thread takes
// 4*kTopkU consecutive entries per round.  A round's selected entries fill a
// contiguous run of the output: they are placed in LDS (`stage`, kEmitStage
// words; any overflow is written directly) and then stored coalesced.
constexpr int kEmitStage = kSelectBins1;
// The score of every emitted entry also goes to the buffer `srs` (a range of
// zero bytes when no scores are wanted, so the stores are dropped): written
// directly, not staged -- a checking aid, not the fast path.
template <int E, int NT, typename Get>
__device__ inline void emit_selected(int cnt, uint32_t T, uint32_t need_eq, uint32_t m, const int32_t* list,
                                     int32_t* out, __amdgpu_buffer_rsrc_t srs, uint32_t* scratch, int32_t* stage,
                                     Get get) {
  const int tid = threadIdx.x;
  const uint32_t need_gt = m - need_eq;
  uint32_t g_gt = 0, g_eq = 0;
  for (int base = 0; base < cnt; base += E * NT) {
    const int i0 = base + tid * E;
    uint32_t key[E];
    int slot[E];
    get(i0, key, slot);  // entries past cnt get slot -1
    uint32_t cgt = 0, ceq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool valid = slot[e] >= 0;
      cgt += (valid && key[e] > T) ? 1u : 0u;
      ceq += (valid && key[e] == T) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t excl = block_exclusive_sum<NT>(cgt | (ceq << 16), scratch, &tot);
    const uint32_t p0 = g_gt + min(g_eq, need_eq);  // the round's first output position
    uint32_t gt_before = g_gt + (excl & 0xFFFFu), eq_before = g_eq + (excl >> 16);
    auto put = [&](uint32_t p, int sl, uint32_t k) {
      if (p >= m) return;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(key_score(k)), srs, (int)(p * 4), 0, 0);
      if (p - p0 < (uint32_t)kEmitStage) stage[p - p0] = sl;
      else out[p] = list ? list[sl] : sl;
    };
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (slot[e] < 0) continue;
      if (key[e] > T) {
        put(gt_before + min(eq_before, need_eq), slot[e], key[e]);
        ++gt_before;
      } else if (key[e] == T) {
        if (eq_before < need_eq) put(gt_before + eq_before, slot[e], key[e]);
        ++eq_before;
      }
    }
    g_gt += tot & 0xFFFFu;
    g_eq += tot >> 16;
    const uint32_t p1 = min(g_gt + min(g_eq, need_eq), m);
    __syncthreads();
    for (uint32_t o = tid; o < min(p1 - p0, (uint32_t)kEmitStage); o += NT) {
      const int sl = stage[o];
      out[p0 + o] = list ? list[sl] : sl;
    }
    __syncthreads();
    if (g_gt >= need_gt && g_eq >= need_eq) break;
  }
}

// LDS of the long-row selection.
struct alignas(16) SelectShared {
  uint32_t hist[1 << kTopkBits1];
  uint32_t ckey[kTopkCap];
  int32_t cslot[kTopkCap];
  uint32_t scratch[kTopkThreads / kWave + 1];  // one word per wave of the largest workgroup
  uint32_t sh_bin, sh_above;
};

// Second half of a long-row selection: the first digit b1 is fixed and rem
// keys are still needed from bin b1.  Finds the remaining 20 bits in two 10-bit
// digits (over the ncand keys staged in LDS in index order, or, for
// ncand < 0, over the row in memory) and emits the selection in index order.
template <int NT = kTopkThreads>
__device__ __forceinline__ void select_finish(SelectShared& sm, int ncand, uint32_t b1, uint32_t rem, const float* row,
                              int n, uint32_t m, const int32_t* list, int32_t* out, float* outs) {
  const int tid = threadIdx.x;
  uint32_t prefix = b1 << (32 - kTopkBits1);
  uint32_t pmask = ~0u << (32 - kTopkBits1);
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    for (int b = tid; b < 1024; b += NT) sm.hist[b] = 0u;
    __syncthreads();
    if (ncand >= 0) {
      for (int c = tid; c < ncand; c += NT) {
        const uint32_t key = sm.ckey[c];
        if ((key & pmask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 1023u], 1u);
      }
    } else {
      for (int base = 0; base < n; base += kTopkU * NT * 4) {
        float4 v[kTopkU];
#pragma unroll
        for (int u = 0; u < kTopkU; ++u) v[u] = load4(row, base + (u * NT + tid) * 4, n);
#pragma unroll
        for (int u = 0; u < kTopkU; ++u) {
          const int s0 = base + (u * NT + tid) * 4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (s0 + e >= n) continue;
            const uint32_t key = score_key(f4(v[u], e));
            if ((key & pmask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 1023u], 1u);
          }
        }
      }
    }
    __syncthreads();
    find_bin<NT>(sm.hist, 1024, rem, sm.scratch, &sm.sh_bin, &sm.sh_above);
    prefix |= sm.sh_bin << shift;
    pmask |= 1023u << shift;
    rem -= sm.sh_above;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t need_eq = rem;  // keys equal to T to take, lowest positions first
  int32_t* stage = reinterpret_cast<int32_t*>(sm.hist);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc(outs ? (void*)outs : (void*)out, 0, outs ? (int)(m * 4) : 0, 0x00020000);
  if (ncand >= 0) {
    // four consecutive staged entries per thread: one 16-byte read each
    emit_selected<4, NT>(ncand, T, need_eq, m, list, out, srs, sm.scratch, stage, [&](int i0, uint32_t* key, int* slot) {
      const uint4 kv = *reinterpret_cast<const uint4*>(&sm.ckey[i0 < kTopkCap ? i0 : 0]);
      const int4 sv = *reinterpret_cast<const int4*>(&sm.cslot[i0 < kTopkCap ? i0 : 0]);
      key[0] = kv.x, key[1] = kv.y, key[2] = kv.z, key[3] = kv.w;
      slot[0] = sv.x, slot[1] = sv.y, slot[2] = sv.z, slot[3] = sv.w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i0 + e >= ncand) slot[e] = -1;
    });
  } else {
    emit_selected<4 * kTopkU, NT>(n, T, need_eq, m, list, out, srs, sm.scratch, stage, [&](int i0, uint32_t* key, int* slot) {
#pragma unroll
      for (int e = 0; e < 4 * kTopkU; ++e) {
        const bool valid = i0 + e < n;
        key[e] = valid ? score_key(row[i0 + e]) : 0u;
        slot[e] = valid ? i0 + e : -1;
      }
    });
  }
}


// ---------------------------------------------------------------------------
// Top-m of short rows (n <= 4096, e.g. a member's candidates): one wave per
// row.  The row's keys live in registers (64 per lane) and the radix select
// runs 8-bit digits against a private 256-bin LDS histogram per wave, starting
// below the bits all of the row's keys share.  After the first digit the keys
// of the threshold bin (usually a few percent of the row) are compacted into
// LDS and the remaining digits run on that short list.  The index-ordered
// emission is a wave-level scan, so no workgroup barrier is needed.  Lane l
// holds elements 256*i + 4*l .. 256*i + 4*l + 3 of chunk i.
// ---------------------------------------------------------------------------
constexpr int kSmallMax = 4096;
constexpr int kSmallWaves = 4;
constexpr int kSmallChunks = kSmallMax / 256;
constexpr int kSmallCand = 512;  // threshold-bin keys a wave compacts for its later digits

__device__ inline uint32_t wave_exclusive_sum(uint32_t v, uint32_t* total) {
  const uint32_t inc = wave_inclusive_sum(v);
  *total = (uint32_t)__builtin_amdgcn_readlane((int)inc, kWave - 1);
  return inc - v;
}

// Maximum over the wave (DPP row shifts and row broadcasts, then lane 63).
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true));   // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true));   // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true));   // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true));   // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// Orders this wave's LDS accesses across lanes (wave-scope fence + barrier).
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// The top-m of one short row by one wave: the scores of slots [0, lmax)
// (lmax <= kSmallMax) in `row`, the positions of the slots in `list`
// (ascending, -1 padded); slots whose position is not in [0, t] are excluded.
// Writes m positions (and their scores if outs is non-null) to out, -1 / NaN
// padded.  cand (kSmallCand words) is this wave's LDS.
__device__ inline void wave_row_select(const float* row, const int32_t* list, int lmax, int t, uint32_t m,
                                       int32_t* out, float* outs, uint32_t* cand) {
  const int lane = threadIdx.x & 63;
  uint32_t key[kSmallChunks * 4];
  int32_t val[kSmallChunks * 4];
  // every load of the row and of its positions is issued before any is used
  // (range-checked buffer loads: no branch, so no wait between them)
  const __amdgpu_buffer_rsrc_t rrow = make_rsrc(row, (uint32_t)lmax * 4u);
  const __amdgpu_buffer_rsrc_t rlist = make_rsrc(list, (uint32_t)lmax * 4u);
  float4 v[kSmallChunks];
  i32x4 p[kSmallChunks];
#pragma unroll
  for (int c = 0; c < kSmallChunks; ++c) {
    const int s0 = c * 256 + lane * 4;
    v[c] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rrow, s0 * 4, 0, 0));
    p[c] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rlist, s0 * 4, 0, 0));
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of their first use
  uint32_t cnt_le = 0;
#pragma unroll
  for (int c = 0; c < kSmallChunks; ++c) {
    const int s0 = c * 256 + lane * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      key[c * 4 + e] = score_key(f4(v[c], e));
      val[c * 4 + e] = p[c][e];
      cnt_le += (s0 + e < lmax && p[c][e] >= 0 && p[c][e] <= t) ? 1u : 0u;
    }
  }
  uint32_t n_u;
  wave_exclusive_sum(cnt_le, &n_u);
  const int n = (int)n_u;
  if (n <= (int)m) {
    for (int s = lane; s < (int)m; s += kWave) {
      out[s] = s < n ? list[s] : -1;
      if (outs) outs[s] = s < n ? row[s] : no_score();
    }
    return;
  }
  // Entries past the row get key 0.  No score has key 0 (it would be a NaN),
  // so they rank below every entry of the row: they never reach the threshold
  // and are never emitted.
  uint32_t kmax = 0u, kmin1 = 0xFFFFFFFFu;  // kmin1: smallest key - 1 of the row
#pragma unroll
  for (int c = 0; c < kSmallChunks; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t k = c * 256 + lane * 4 + e < n ? key[c * 4 + e] : 0u;
      key[c * 4 + e] = k;
      kmax = max(kmax, k);
      kmin1 = min(kmin1, k - 1u);
    }
  kmax = wave_max_u32(kmax);
  const uint32_t kmin = ~wave_max_u32(~kmin1) + 1u;
  // bits above the highest bit where the row's keys differ are common to all
  const int top = kmin == kmax ? 0 : 32 - __clz((int)(kmin ^ kmax));  // undetermined low bits
  const uint32_t pmask = top == 32 ? 0u : ~0u << top;

  // T, the m-th largest key, by a binary search over the undetermined bits,
  // most significant first: T takes bit b when at least m keys are >= T | 2^b.
  // `above` counts the keys >= T + 2^(b+1) (fewer than m) and `inwin` those in
  // [T, T + 2^(b+1)), the keys not yet decided.  Counting is a compare and an
  // add per key and a wave sum per bit (no atomics); it runs over the
  // registers until the undecided keys fit the wave's LDS list, then over
  // that list.  At the end `above` counts the keys > T.
  uint32_t T = kmax & pmask, above = 0, inwin = (uint32_t)n;
  int b = top - 1;
  bool narrowed = false;
  while (b >= 0 && inwin > (uint32_t)kSmallCand) {
    const uint32_t Tc = T | (1u << b);
    // four independent partial counts, so that each compare's lane mask is
    // consumed a few instructions later rather than by the next one
    uint32_t c4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < kSmallChunks * 4; ++j) c4[j & 3] += key[j] >= Tc ? 1u : 0u;
    uint32_t c = (c4[0] + c4[1]) + (c4[2] + c4[3]);
    wave_exclusive_sum(c, &c);
    if (c >= m) {
      T = Tc;
      inwin = c - above;
    } else {
      inwin = above + inwin - c;
      above = c;
    }
    --b;
    if (!narrowed && b >= 0) {
      // The first bit usually sets apart a few outlying keys; the rest then
      // share several more leading bits, which one min/max pass over the
      // undecided keys skips at once (the range they span never holds a key
      // outside them, so `above` and `inwin` stay as they are).
      narrowed = true;
      const uint32_t wmask = ~0u << (b + 1);  // b + 1 <= 31 here
      uint32_t hi = 0u, nlo = 0u;             // largest key, complement of the smallest
#pragma unroll
      for (int j = 0; j < kSmallChunks * 4; ++j) {
        const bool in = key[j] != 0u && (key[j] & wmask) == T;
        hi = max(hi, in ? key[j] : 0u);
        nlo = max(nlo, in ? ~key[j] : 0u);
      }
      hi = wave_max_u32(hi);
      const uint32_t lo = ~wave_max_u32(nlo);
      const int t2 = hi == lo ? 0 : 32 - __clz((int)(hi ^ lo));
      if (t2 < b + 1) {
        T = t2 == 0 ? hi : hi & (~0u << t2);
        b = t2 - 1;
      }
    }
  }
  if (b >= 0) {
    // compact the undecided keys (any order: only their values matter); a
    // valid key is never 0, so the entries past the row stay out
    const uint32_t wmask = b + 1 >= 32 ? 0u : ~0u << (b + 1);
    uint32_t base = 0;
#pragma unroll
    for (int j = 0; j < kSmallChunks * 4; ++j) {
      const bool hit = key[j] != 0u && (key[j] & wmask) == T;
      const unsigned long long mk = __ballot(hit);
      if (hit) cand[base + __builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u))] = key[j];
      base += (uint32_t)__popcll(mk);
    }
    wave_sync();
    uint32_t ck[kSmallCand / kWave];
#pragma unroll
    for (int j = 0; j < kSmallCand / kWave; ++j) ck[j] = (uint32_t)(j * kWave + lane) < base ? cand[j * kWave + lane] : 0u;
    wave_sync();
    const uint32_t base_above = above;  // keys above the list's range
    for (; b >= 0; --b) {
      const uint32_t Tc = T | (1u << b);
      uint32_t c = 0;
#pragma unroll
      for (int j = 0; j < kSmallCand / kWave; ++j) c += ck[j] >= Tc ? 1u : 0u;
      wave_exclusive_sum(c, &c);
      c += base_above;
      if (c >= m)
        T = Tc;
      else
        above = c;
    }
  }
  const uint32_t need_eq = m - above;

  // emission in index order (entries past the row hold key 0 < T).  No
  // branch per entry: every entry's store is issued, the unselected ones at
  // an offset past the row's range, which the buffer range check drops.
  const __amdgpu_buffer_rsrc_t rout = make_rsrc(out, m * 4u);
  const __amdgpu_buffer_rsrc_t routs = make_rsrc(outs, outs ? m * 4u : 0u);
  uint32_t g_gt = 0, g_eq = 0;
#pragma unroll
  for (int c = 0; c < kSmallChunks; ++c) {
    uint32_t cgt = 0, ceq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cgt += key[c * 4 + e] > T ? 1u : 0u;
      ceq += key[c * 4 + e] == T ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t excl = wave_exclusive_sum(cgt | (ceq << 16), &tot);
    uint32_t gt_before = g_gt + (excl & 0xFFFFu), eq_before = g_eq + (excl >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t kk = key[c * 4 + e];
      const bool gt = kk > T, eq = kk == T;
      // a key above T goes after every earlier key above T and the first
      // need_eq keys equal to T; a key equal to T is taken while fewer than
      // need_eq equal keys precede it
      const uint32_t p = gt ? gt_before + min(eq_before, need_eq) : gt_before + eq_before;
      const uint32_t off = (gt || (eq && eq_before < need_eq)) ? p * 4u : m * 4u;
      __builtin_amdgcn_raw_buffer_store_b32((uint32_t)val[c * 4 + e], rout, (int)off, 0, 0);
      if (outs) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(key_score(kk)), routs, (int)off, 0, 0);
      gt_before += gt ? 1u : 0u;
      eq_before += eq ? 1u : 0u;
    }
    g_gt += tot & 0xFFFFu;
    g_eq += tot >> 16;
  }
}

}  // namespace pivot
