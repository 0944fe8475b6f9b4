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
// Two kernels:
//  * score_block_kernel: 8 query rows per workgroup (one wave each) share key
//                        tiles staged in LDS.  Full-prefix scan: contiguous
//                        keys, row r keeps keys <= pos(r).  Refine: the members
//                        of one group score the group's candidate keys,
//                        gathered from the key cache through its candidate list.
//  * decode_scan_kernel: one sequence's 1-2 query rows stream that sequence's
//                        key cache through per-wave LDS rings filled by
//                        direct-to-LDS loads (no reuse across rows to stage).
#pragma once

#include "pivot_device.h"
#include "pivot_kernels.h"

#ifndef PIVOT_SCAN_SCHED
#define PIVOT_SCAN_SCHED 1
#endif

namespace pivot {

constexpr int kScanRows = 8;      // query rows (waves) per scoring workgroup
constexpr int kRefineSlotMax = kRefineSlotLimit;  // candidate slots per Refine workgroup
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

template <int HB>
struct TileAcc {
  f32x16 v[HB];
};

// Contract one 32-key tile whose B fragments are produced by `bfrag(ks)`:
// acc.v[mb][i] = q[head(mb, i, lane)] . k[tile + lane % 32].
template <int DT, int D, int HB, typename BF>
__device__ inline void mma_tile(const QueryRegs<DT, D, HB>& qr, BF bfrag, TileAcc<HB>& acc) {
  constexpr int NKS = D / Fmt<DT>::KSTEP;
#pragma unroll
  for (int mb = 0; mb < HB; ++mb) acc.v[mb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const typename Fmt<DT>::frag b = bfrag(ks);
#pragma unroll
    for (int mb = 0; mb < HB; ++mb) acc.v[mb] = Fmt<DT>::mma(qr.a[mb][ks], b, acc.v[mb]);
  }
}

// max(0, x) on the bits of a finite float: every negative float (and -0) has
// a negative signed-integer pattern, so an integer max with 0 gives +0 there
// and leaves non-negative values unchanged.  One integer op, which (unlike a
// float max) needs no NaN-quieting of the matrix-core result first.
__device__ inline float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Per-lane part of ReLU, head weights and head sum of one contracted tile:
// the sum over the 16*HB heads this lane holds for its key column.
template <int DT, int D, int HB>
__device__ inline float tile_partial(const QueryRegs<DT, D, HB>& qr, const TileAcc<HB>& acc) {
  float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
  for (int mb = 0; mb < HB; ++mb) {
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      p0 = fmaf(qr.wv[mb][i + 0], relu(acc.v[mb][i + 0]), p0);
      p1 = fmaf(qr.wv[mb][i + 1], relu(acc.v[mb][i + 1]), p1);
      p2 = fmaf(qr.wv[mb][i + 2], relu(acc.v[mb][i + 2]), p2);
      p3 = fmaf(qr.wv[mb][i + 3], relu(acc.v[mb][i + 3]), p3);
    }
  }
  return (p0 + p1) + (p2 + p3);
}

// Finish two tiles at once: the two lane halves hold the other half of the
// heads, so one lane-half swap (rows of 32 lanes) plus one add leaves tile A's
// 32 scores in lanes 0..31 and tile B's in lanes 32..63.
__device__ inline float pair_combine(float pa, float pb) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(pa), __float_as_uint(pb), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One tile: every lane ends with the score of key (tile + lane % 32).
template <int DT, int D, int HB>
__device__ inline float tile_epilogue(const QueryRegs<DT, D, HB>& qr, const TileAcc<HB>& acc) {
  const float p = tile_partial<DT, D, HB>(qr, acc);
  return pair_combine(p, p);
}

template <int DT, int D, int HB, typename BF>
__device__ inline float score_tile(const QueryRegs<DT, D, HB>& qr, BF bfrag) {
  TileAcc<HB> acc;
  mma_tile<DT, D, HB>(qr, bfrag, acc);
  return tile_epilogue<DT, D, HB>(qr, acc);
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
//
// A workgroup = 8 waves = 8 consecutive query rows, over a chunk of kc keys.
// Keys are staged in LDS in stages of ST tiles of 32 keys (double buffered:
// the next stage is loaded into registers during the current one and stored
// to LDS at its end, one barrier per stage).  Within a stage each wave runs a
// fixed software pipeline over the tiles, with the B fragments of tile t+1
// read from LDS while tile t is contracted, and the epilogue of tile t-1
// interleaved with the contraction of tile t:
//   even tile t: contract; finish and store the pair (t-2, t-1), which for
//                t = 0 is the previous stage's last pair
//   odd tile t:  contract; partial of tile t-1
// Every tile of a stage is contracted; stores beyond a row's causal limit
// (or the chunk end) fall outside the row's buffer range and are dropped by
// the hardware range check, so the stage body has no data-dependent branch.
// ---------------------------------------------------------------------------
constexpr int kScanStageTiles = 8;    // full-prefix scan: fewer barriers per key
constexpr int kRefineStageTiles = 4;  // Refine: chunks of candidate slots are short

// Interleaving hint for one tile step: the DS reads of the next tile, the 16
// contractions and the previous tile's epilogue alternate.
__device__ inline void sched_tile_step() {
#if PIVOT_SCAN_SCHED
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
  }
#endif
}

constexpr int kScanWaveThreads = kScanRows * kWave;

// Geometry of one workgroup of the scoring loop (ROWS waves, one query row
// each): its query rows, the key positions it covers and where scores go.
//  * full-prefix scan (GATHER = false, ScanArgs): rows rb..rb+ROWS-1, a chunk of
//    contiguous keys [k0, k1); row r keeps keys <= pos(r).
//  * Refine (GATHER = true, RefineArgs): the members of one group, a chunk of
//    candidate slots [k0, k1) whose keys are gathered through the group's
//    candidate list; every slot < the group's candidate count is kept.
template <int DT, int D, int HB, bool GATHER, int ROWS, typename Args>
__global__ __launch_bounds__(ROWS * kWave) void score_block_kernel(Args a) {
  using KT = KeyTile<DT, D>;
  using Frag = typename Fmt<DT>::frag;
  constexpr int NT = ROWS * kWave;
  constexpr int NKS = D / Fmt<DT>::KSTEP;
  // tiles per stage: the preferred count where two stages fit in LDS
  constexpr int ST_PREF = GATHER ? kRefineStageTiles : kScanStageTiles;
  constexpr int ST = 2 * ST_PREF * KT::BYTES <= 150 * 1024 ? ST_PREF : 4;
  constexpr int SCH = ST * KT::CHUNKS;  // 16-byte pieces per stage
  constexpr int NPT = (SCH + NT - 1) / NT;
  constexpr int STAGE_BYTES = ST * KT::BYTES;
  constexpr int STAGE_KEYS = ST * kTileN;
  constexpr int RCH = KT::ROW / 16;  // 16-byte pieces per key row
  static_assert(ST % 2 == 0, "the pipeline below works on pairs of tiles");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE_BYTES];
  __shared__ int32_t cand_s[GATHER ? kRefineSlotMax : 1];  // Refine: positions of slots [k0, k1)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- workgroup geometry ----
  int k0, k1;                 // key positions (scan) or candidate slots (Refine)
  int r;                      // this wave's query row
  bool active;                // the row exists
  int nvalid;                 // scores [0, nvalid) of the row are stored
  long long srow_index;       // row of S
  __amdgpu_buffer_rsrc_t krs; // keys: the chunk (scan) or the whole key array (Refine)
  __amdgpu_buffer_rsrc_t crs; // Refine: candidate positions of slots [k0, k1)
  __amdgpu_buffer_rsrc_t ksr; // fp8 key scales (empty for bf16)
  int gj = 0;                 // Refine: this workgroup's group
  if constexpr (!GATHER) {
    // XCD-aware order: workgroups are dealt to the chip's eight XCDs in turn
    // (linear id i goes to XCD i % 8), so the i-th workgroup takes the
    // (i % 8) * n/8 + i/8 -th (chunk, row block) in chunk-major order: the
    // workgroups on one XCD work through consecutive row blocks of the same
    // key chunk together and read its keys through that XCD's L2
    const int per = gridDim.x / 8;
    const int lin = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (lin >= a.nchunks * a.nblocks) return;
    const int bx = lin / a.nblocks, by = lin % a.nblocks;
    const int rb = a.row_begin + by * ROWS;
    const int rlast = min(rb + ROWS, a.row_end) - 1;
    const int lim = min(rlast * a.pos_mul + a.pos_add, a.pos_cap) + 1;  // keys 0..lim-1
    k0 = bx * a.kc;
    if (k0 >= lim) return;
    k1 = min(k0 + a.kc, lim);
    r = rb + wid;
    active = r <= rlast;
    const int pos = active ? min(r * a.pos_mul + a.pos_add, a.pos_cap) : -1;
    nvalid = active ? max(0, min(pos + 1, k1)) : 0;  // a row may see no key at all
    srow_index = active ? r - a.row_begin : 0;
    krs = make_rsrc(a.k + (size_t)k0 * KT::ROW, (uint32_t)(k1 - k0) * KT::ROW);
    crs = krs;
    ksr = make_rsrc(DT == kFP8 ? a.k_scale + k0 : a.S, DT == kFP8 ? (uint32_t)(k1 - k0) * 4u : 0u);
  } else {
    const int bx = blockIdx.x, bz = blockIdx.z;
    gj = a.grp_begin + blockIdx.y;
    const int j = gj;
    int row0, nmem, ncand, nkeys;
    size_t keybase = 0;
    if (a.kind == 0) {
      row0 = j * a.g;
      nmem = min(a.g, a.L - row0);
      ncand = min(a.m, max(0, row0 + nmem - a.excl));  // min(m, e_j + 1 - excl)
      nkeys = a.L;
    } else {
      const int nb = a.cache_len[j];
      if (nb < a.g || nb > a.Lmax) return;
      row0 = j * a.g;
      nmem = a.g;
      ncand = min(a.m, max(0, nb - a.excl));
      nkeys = a.bt ? a.pool_rows : nb;  // paged: the whole pool, slots translated below
      keybase = a.bt ? 0 : (size_t)j * a.Lmax;
    }
    k0 = bx * a.slot_chunk;
    if (k0 >= ncand) return;
    k1 = min(k0 + a.slot_chunk, ncand);
    const int mem = bz * ROWS + wid;
    active = mem < nmem;
    r = row0 + (active ? mem : 0);
    nvalid = active ? k1 : 0;
    srow_index = r - a.row_base;
    krs = make_rsrc(a.k + keybase * KT::ROW, (uint32_t)nkeys * KT::ROW);
    crs = make_rsrc(a.cand + (size_t)(j - a.grp_begin) * a.ldc + k0, (uint32_t)(k1 - k0) * 4u);
    ksr = make_rsrc(DT == kFP8 ? a.k_scale + keybase : a.q_scale, DT == kFP8 ? (uint32_t)nkeys * 4u : 0u);
  }
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.S + srow_index * a.ldS, (uint32_t)nvalid * 4u);

  QueryRegs<DT, D, HB> qr;
  float qs = 1.f;
  if (active) {
    qr.load(a.q + (size_t)r * a.H * D * Fmt<DT>::ESZ, a.w + (size_t)r * a.H, a.H, lane);
    if constexpr (DT == kFP8) qs = a.q_scale[r];
  } else {
#pragma unroll
    for (int mb = 0; mb < HB; ++mb) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qr.a[mb][ks] = zero_frag<DT>();
#pragma unroll
      for (int i = 0; i < 16; ++i) qr.wv[mb][i] = 0.f;
    }
  }

  // key row of slot `slot` (Refine) -- 0 outside the workgroup's slots.  With
  // a paged cache the candidate positions become pool rows here; a page id
  // outside the pool gives the row just past it, which reads as zeros.
  if constexpr (GATHER) {
    // the chunk's positions are loaded in batches of 8 per thread, every load
    // of a batch issued before any is used (one memory latency per 8 NT
    // positions, not per NT); slots past the chunk read as 0 through the
    // range check and are not stored
    constexpr int CB = 8;
    for (int base = 0; base < k1 - k0; base += CB * NT) {
      int cv[CB];
#pragma unroll
      for (int i = 0; i < CB; ++i)
        cv[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(crs, (base + tid + i * NT) * 4, 0, 0);
      if constexpr (std::is_same_v<Args, RefineArgs>) {
        if (a.bt) {
          const int j = gj;
#pragma unroll
          for (int i = 0; i < CB; ++i) {
            const int v = max(cv[i], 0);
            const int pg = a.bt[(size_t)j * a.bt_stride + (v >> a.page_shift)];
            cv[i] = (unsigned)pg < (unsigned)(a.pool_rows >> a.page_shift)
                        ? (pg << a.page_shift) + (v & ((1 << a.page_shift) - 1))
                        : a.pool_rows;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < CB; ++i)
        if (base + tid + i * NT < k1 - k0) cand_s[base + tid + i * NT] = cv[i];
    }
    __syncthreads();
  }
  auto cand_pos = [&](int slot) -> int {
    const int r = slot - k0;
    const int v = cand_s[(unsigned)r < (unsigned)(k1 - k0) ? r : 0];
    return (unsigned)r < (unsigned)(k1 - k0) ? v : 0;
  };

  i32x4 pre[NPT];
  auto fetch = [&](int base) {  // stage starting at key/slot `base` -> registers
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int c = tid + i * NT;
      if (SCH % NT == 0 || c < SCH) {
        int off;
        if constexpr (!GATHER)
          off = (base - k0) * KT::ROW + c * 16;
        else
          off = (int)((uint32_t)cand_pos(base + c / RCH) * KT::ROW + (c % RCH) * 16);
        pre[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
      }
    }
  };
  auto stash = [&](int buf) {
    uint8_t* st = lds + buf * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int c = tid + i * NT;
      if (SCH % NT == 0 || c < SCH)
        *reinterpret_cast<i32x4*>(st + (c / RCH) * KT::STRIDE + (c % RCH) * 16) = pre[i];
    }
  };

  const int hf = lane >> 5, n = lane & 31;
  auto load_b = [&](const uint8_t* st, int tt, Frag* b) {
    const uint8_t* brow = st + (tt * kTileN + n) * KT::STRIDE;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) b[ks] = load_frag<DT>(brow + frag_offset<DT, D>(ks, hf));
  };
  auto contract = [&](const Frag* b, TileAcc<HB>& acc) {
    mma_tile<DT, D, HB>(qr, [&](int ks) { return b[ks]; }, acc);
  };
  // pair of tiles starting at key/slot t0: lane l holds t0 + l
  auto store_pair = [&](float pa, float pb, int t0) {
    float s = pair_combine(pa, pb);
    const int key = t0 + lane;
    if constexpr (DT == kFP8) {
      const int kp = GATHER ? cand_pos(key) : key - k0;
      s = (s * qs) * __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ksr, kp * 4, 0, 0));
    }
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), srs, key * 4, 0, 0);
  };

  fetch(k0);
  stash(0);
  __syncthreads();
  fetch(k0 + STAGE_KEYS);

  // The stage body has no branch: on the first stage the "previous pair" is
  // sent to slot -2^28 (the byte offset wraps far past every row's range),
  // and past the chunk's last stage the prefetch reads beyond the key range
  // (Refine: slots past the list read candidate 0); the buffer range checks
  // drop the former and make the latter harmless.
  TileAcc<HB> acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mb = 0; mb < HB; ++mb) acc[t].v[mb] = f32x16{};
  Frag b0[NKS], b1[NKS];
  float pa = 0.f;
  int buf = 0;
  for (int sb = k0; sb < k1; sb += STAGE_KEYS) {
    const uint8_t* st = lds + buf * STAGE_BYTES;
    load_b(st, 0, b0);
#if PIVOT_SCAN_SCHED
    // Refine and fp8: all of the first tile's fragment reads go out together
    // right after the barrier (the stage was not readable before it), rather
    // than each just ahead of the contraction that uses it.  (The bf16
    // full-prefix scan has no registers to spare for this: it would spill.)
    if constexpr (GATHER || DT == kFP8) __builtin_amdgcn_sched_barrier(0);
#endif
#pragma unroll
    for (int t = 0; t < ST; t += 2) {
      // even tile: contract it, finish and store the pair before it
      load_b(st, t + 1, b1);
      contract(b0, acc[0]);
      const int prev = t > 0 ? sb + (t - 2) * kTileN : sb != k0 ? sb - 2 * kTileN : -(1 << 28);
      store_pair(pa, tile_partial<DT, D, HB>(qr, acc[1]), prev);
      sched_tile_step();
      // odd tile: contract it, partial of the even tile
      if (t + 2 < ST) load_b(st, t + 2, b0);
      contract(b1, acc[1]);
      pa = tile_partial<DT, D, HB>(qr, acc[0]);
      sched_tile_step();
    }
    stash(buf ^ 1);
    fetch(sb + 2 * STAGE_KEYS);
    __syncthreads();
    buf ^= 1;
  }
  // the last stage's last pair
  const int last = k0 + ((k1 - k0 - 1) / STAGE_KEYS) * STAGE_KEYS;
  store_pair(pa, tile_partial<DT, D, HB>(qr, acc[1]), last + (ST - 2) * kTileN);
}

// ---------------------------------------------------------------------------
// Decode scan: QR query rows of one sequence stream its key cache.
//
// The batch's keys are cut into pairs of 32-key tiles, sequence by sequence,
// and every workgroup takes an equal run of consecutive pairs (a run spans at
// most a few sequences).  Inside a run the waves take turns at blocks of four
// consecutive pairs; each wave streams its pairs through a ring of R stages of
// its own in LDS, filled by direct-to-LDS buffer loads (no registers held by
// loads in flight): while one stage is contracted the other R-1 are loading.  A stage is written in 1 KB wave-wide pieces,
// 16 bytes per lane, with the 16-byte chunks of each key row XOR-swizzled by
// the row index so that the fragment reads of 32 rows spread over the banks.
// The buffer range ends at the run's last key (reads beyond it return zero,
// stores beyond a row's causal limit are dropped).  A block's 256 scores are
// collected in LDS and written with one 16-byte-per-lane store, and the top 12
// bits of their keys are histogrammed per row in LDS and added to the row's
// histogram in memory whenever the run moves to the next sequence.
//
// With a paged cache (PAGED) a pair of tiles lies inside one page: each pair's
// loads get a descriptor of their own, based at the pair's first key in its
// page and ranged to the run's last key, from a page id read through the
// scalar cache.
// ---------------------------------------------------------------------------
template <int DT, int D, int QR>
struct DecGeom {
  static constexpr int ROW = D * Fmt<DT>::ESZ;            // bytes of one key row
  static constexpr int PAIR_KEYS = 2 * kTileN;
  static constexpr int PAIR_BYTES = PAIR_KEYS * ROW;
  static constexpr int STAGE_BYTES = PAIR_BYTES + (DT == kFP8 ? PAIR_KEYS * 4 : 0);  // + key scales
  static constexpr int BLOCK_PAIRS = 4;                   // pairs whose scores are stored together
  static constexpr int FIXED_W = QR * BLOCK_PAIRS * PAIR_KEYS * 4;  // per-wave score block
  static constexpr bool fits(int w, int r) {
    return r * w * STAGE_BYTES + w * FIXED_W + QR * kSelectBins1 * 4 + 1024 <= 158 * 1024;
  }
  static constexpr int LOADS = PAIR_BYTES / 1024;         // wave-wide 1 KB pieces per pair
  static constexpr int STAGE_OPS = LOADS + (DT == kFP8 ? 1 : 0);  // loads that fill one stage
  // two waves per SIMD when their rings fit (their compute overlaps), else one
  static constexpr int W = fits(8, 2) ? 8 : (fits(4, 3) || fits(4, 2)) ? 4 : (fits(2, 3) || fits(2, 2)) ? 2 : 1;
  // a wait names the newer stages' loads in a 6-bit count
  static constexpr int R = (fits(W, 3) && 2 * STAGE_OPS < 64) ? 3 : 2;
  static constexpr int THREADS = W * kWave;
  static constexpr int CPR = ROW / 16;                    // 16-byte chunks per key row
  static constexpr int SWM = (CPR < 8 ? CPR : 8) - 1;     // swizzle mask
  static_assert(PAIR_BYTES % 1024 == 0 && fits(W, R) && (R - 1) * STAGE_OPS < 64);
};

// A page id, read with a scalar load: the address is wave-uniform and the
// block table is not written while the kernel runs.
__device__ inline int page_id(const int32_t* bt, size_t i) {
  typedef __attribute__((address_space(4))) const int32_t cint;
  return __builtin_amdgcn_readfirstlane(((cint*)bt)[i]);
}

template <int DT, int D, int HB, int QR, bool PAGED>
__global__ __launch_bounds__((DecGeom<DT, D, QR>::THREADS)) void decode_scan_kernel(DecScanArgs a) {
  using G = DecGeom<DT, D, QR>;
  using Frag = typename Fmt<DT>::frag;
  constexpr int ROW = G::ROW, W = G::W, R = G::R, NT = G::THREADS;
  constexpr int NB = kSelectBins1;
  __shared__ __attribute__((aligned(16))) uint8_t ring0[W][G::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[W][G::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[R > 2 ? W : 1][R > 2 ? G::STAGE_BYTES : 16];
  __shared__ uint32_t hist[QR][NB];
  __shared__ __attribute__((aligned(16))) float sbuf[W][QR][G::BLOCK_PAIRS * G::PAIR_KEYS];
  __shared__ int sh_b, sh_off;
  __shared__ uint32_t sh_lo, sh_hi;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, n = lane & 31;
  const int ri0 = blockIdx.z * QR;

  auto seq_pairs = [&](int b) -> uint32_t {
    const int nb = a.cache_len[b];
    return (nb < a.g || nb > a.Lmax) ? 0u : (uint32_t)(nb + G::PAIR_KEYS - 1) / G::PAIR_KEYS;
  };
  // Runs are cut in work units: every non-empty sequence counts its pairs plus
  // kDecSegmentPairs units for the set-up of a segment (query rows, the ring's
  // first stages, the histogram flush), which stand for no keys.  A run that
  // reaches into a further sequence thus takes correspondingly fewer pairs,
  // and the workgroups finish together.
  constexpr uint32_t SEG = kDecSegmentPairs;
  auto seq_units = [&](int b) -> uint32_t {
    const uint32_t p = seq_pairs(b);
    return p ? p + SEG : 0u;
  };
  // this workgroup's run [lo, hi) of the batch's work units and where it
  // starts, found by the first wave alone (prefix sums over the sequences, a
  // wave's width at a time) while the others clear the histograms
  if (wid == 0) {
    uint32_t total = 0;
    for (int b0 = 0; b0 < a.B; b0 += kWave) {
      const uint32_t inc = wave_inclusive_sum(b0 + lane < a.B ? seq_units(b0 + lane) : 0u);
      total += (uint32_t)__builtin_amdgcn_readlane((int)inc, kWave - 1);
    }
    const uint32_t lo_ = (uint32_t)((uint64_t)total * blockIdx.x / gridDim.x);
    const uint32_t hi_ = (uint32_t)((uint64_t)total * (blockIdx.x + 1) / gridDim.x);
    uint32_t base = 0;
    for (int b0 = 0; b0 < a.B && base <= lo_; b0 += kWave) {
      const int bb = b0 + lane;
      const uint32_t p = bb < a.B ? seq_units(bb) : 0u;
      const uint32_t inc = wave_inclusive_sum(p);
      const uint32_t ex = inc - p;
      if (p && base + ex <= lo_ && lo_ < base + ex + p) {
        sh_b = bb;
        sh_off = (int)(lo_ - base - ex);
      }
      base += (uint32_t)__builtin_amdgcn_readlane((int)inc, kWave - 1);
    }
    if (lane == 0) {
      sh_lo = lo_;
      sh_hi = hi_;
    }
  }
  for (int i = 0; i < QR; ++i)
    for (int e = tid; e < NB; e += NT) hist[i][e] = 0u;
  __syncthreads();
  const uint32_t lo = sh_lo, hi = sh_hi;
  if (lo == hi) return;
  int b = __builtin_amdgcn_readfirstlane(sh_b);
  uint32_t vo = (uint32_t)__builtin_amdgcn_readfirstlane(sh_off);  // units into sequence b
  uint32_t left = hi - lo;

  while (left > 0 && b < a.B) {
    const int nb = a.cache_len[b];
    const uint32_t take = min(seq_units(b) - vo, left);  // this sequence's units in the run
    const int off = (int)(vo > SEG ? vo - SEG : 0u);     // its first pair
    const int np = (int)(vo + take > SEG ? vo + take - SEG : 0u) - off;
    left -= take;
    vo = 0;
    if (np <= 0) {  // the run holds only set-up units of this sequence
      while (left > 0 && ++b < a.B && seq_pairs(b) == 0) {
      }
      continue;
    }
    const int k0 = off * G::PAIR_KEYS;
    const int k1 = min(k0 + np * G::PAIR_KEYS, nb);

    QueryRegs<DT, D, HB> q[QR];
    float qs[QR];
    int pos[QR];
    __amdgpu_buffer_rsrc_t srs[QR];
    i32x4 krs{}, ksr{};
    if constexpr (!PAGED) {
      krs = dma_rsrc(a.k + ((size_t)b * a.Lmax + k0) * ROW, (uint32_t)(k1 - k0) * ROW, kBufferFlags);
      ksr = dma_rsrc(DT == kFP8 ? (const void*)(a.k_scale + (size_t)b * a.Lmax + k0) : (const void*)a.w,
                     DT == kFP8 ? (uint32_t)(k1 - k0) * 4u : 0u, kBufferFlags);
    }

    // wave-local pair s is pair s % 4 of the wave's block s / 4, i.e. the
    // segment's pair 4 * (wid + W * (s / 4)) + s % 4; stage s % R holds it
    auto pair_of = [&](int s) { return G::BLOCK_PAIRS * (wid + W * (s / G::BLOCK_PAIRS)) + s % G::BLOCK_PAIRS; };
    auto issue = [&](const uint8_t* stage, int s) {
      int key0 = pair_of(s) * G::PAIR_KEYS;
      i32x4 rk = krs, rs = ksr;
      if constexpr (PAGED) {
        // the pair's own descriptors: empty past the run's last key or for a
        // page id outside the pool (the loads then write zeros)
        const int p0 = k0 + key0;
        const uint8_t* kb = a.k;
        const float* sb = DT == kFP8 ? a.k_scale : a.w;
        uint32_t nk = 0;
        if (p0 < k1) {
          const int pg = page_id(a.bt, (size_t)b * a.bt_stride + (p0 >> a.page_shift));
          if ((unsigned)pg < (unsigned)a.num_pages) {
            const size_t row = ((size_t)pg << a.page_shift) + (p0 & ((1 << a.page_shift) - 1));
            kb += row * ROW;
            if constexpr (DT == kFP8) sb += row;
            nk = (uint32_t)min(G::PAIR_KEYS, k1 - p0);
          }
        }
        rk = dma_rsrc(kb, nk * ROW, kBufferFlags);
        rs = dma_rsrc(sb, DT == kFP8 ? nk * 4u : 0u, kBufferFlags);
        key0 = 0;
      }
      const uint32_t dst = lds_addr(stage);
#pragma unroll
      for (int c = 0; c < G::LOADS; ++c) {
        const int slot = c * kWave + lane;
        const int kr = slot / G::CPR;
        const int chunk = (slot % G::CPR) ^ (kr & G::SWM);
        lds_dma16(rk, dst + c * 1024, (uint32_t)((key0 + kr) * ROW + chunk * 16));
      }
      if constexpr (DT == kFP8) lds_dma4(rs, dst + G::PAIR_BYTES, (uint32_t)((key0 + lane) * 4));
    };
    // a stage is complete once at most the R-1 newer stages' loads (and
    // any score stores issued after it) are outstanding
    constexpr int kStageOps = G::STAGE_OPS;
    auto frag_at = [&](const uint8_t* stage, int t, int ks) -> Frag {
      const int kr = t * kTileN + n;
      const int c0 = frag_offset<DT, D>(ks, hf) / 16;
      const uint8_t* row = stage + kr * ROW;
      if constexpr (DT == kBF16) {
        return *reinterpret_cast<const i32x4*>(row + ((c0 ^ (kr & G::SWM)) << 4));
      } else {
        const i32x4 lo4 = *reinterpret_cast<const i32x4*>(row + ((c0 ^ (kr & G::SWM)) << 4));
        const i32x4 hi4 = *reinterpret_cast<const i32x4*>(row + (((c0 + 1) ^ (kr & G::SWM)) << 4));
        return i32x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      }
    };
    auto compute = [&](const uint8_t* stage, int s) {
      const int key = k0 + pair_of(s) * G::PAIR_KEYS + lane;
      const int u = s % G::BLOCK_PAIRS;
      float ksv = 1.f;
      if constexpr (DT == kFP8) ksv = *reinterpret_cast<const float*>(stage + G::PAIR_BYTES + 4 * lane);
#pragma unroll
      for (int i = 0; i < QR; ++i) {
        if (pos[i] < 0) continue;
        TileAcc<HB> acc0, acc1;
        mma_tile<DT, D, HB>(q[i], [&](int ks) { return frag_at(stage, 0, ks); }, acc0);
        mma_tile<DT, D, HB>(q[i], [&](int ks) { return frag_at(stage, 1, ks); }, acc1);
        float sc = pair_combine(tile_partial<DT, D, HB>(q[i], acc0), tile_partial<DT, D, HB>(q[i], acc1));
        if constexpr (DT == kFP8) sc = (sc * qs[i]) * ksv;
        sbuf[wid][i][u * G::PAIR_KEYS + lane] = sc;
        if (a.hist && key < k1 && key <= pos[i]) atomicAdd(&hist[i][score_key(sc) >> 20], 1u);
        if (u == G::BLOCK_PAIRS - 1) {
          const int bkey = key - lane - (G::BLOCK_PAIRS - 1) * G::PAIR_KEYS;
          const float4 v = *reinterpret_cast<const float4*>(&sbuf[wid][i][4 * lane]);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), srs[i], (bkey + 4 * lane) * 4, 0, 0);
        }
      }
    };

    // whole blocks per wave; loads past the segment's last pair read zeros
    const int nblk = (np + G::BLOCK_PAIRS - 1) / G::BLOCK_PAIRS;
    const int npw = nblk > wid ? G::BLOCK_PAIRS * ((nblk - wid + W - 1) / W) : 0;
    // the ring starts filling before the query rows are loaded, so that the
    // two latencies overlap
    issue(ring0[wid], 0);
    issue(ring1[wid], 1);
    if constexpr (R > 2) issue(ring2[wid], 2);
#pragma unroll
    for (int i = 0; i < QR; ++i) {
      const int ri = ri0 + i;
      pos[i] = -1;
      qs[i] = 1.f;
      if (ri < a.qr) {
        const size_t rowi = (size_t)b * a.qr + ri;
        q[i].load(a.q + rowi * a.H * ROW, a.w + rowi * a.H, a.H, lane);
        if constexpr (DT == kFP8) qs[i] = a.q_scale[rowi];
        pos[i] = (a.qr == 1 ? nb - 1 : nb - a.g + ri) - a.excl;
      }
      // whole 16-byte pieces (the row stride is a multiple of 64 keys): the
      // up-to-3 scores past the causal limit that this lets through are unused
      const int nvalid = pos[i] < 0 ? 0 : (min(pos[i] + 1, k1) + 3) & ~3;
      srs[i] = make_rsrc(a.S + ((size_t)b * a.qr + (pos[i] < 0 ? 0 : ri)) * a.ldS, (uint32_t)nvalid * 4u);
    }
    // the query registers are complete (and with them the ring's first
    // stages) before the first contraction
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    for (int s = 0; s < npw; s += R) {
      lds_dma_wait<(R - 1) * kStageOps>();
      compute(ring0[wid], s);
      issue(ring0[wid], s + R);
      lds_dma_wait<(R - 1) * kStageOps>();
      if (s + 1 < npw) compute(ring1[wid], s + 1);
      issue(ring1[wid], s + 1 + R);
      if constexpr (R > 2) {
        lds_dma_wait<(R - 1) * kStageOps>();
        if (s + 2 < npw) compute(ring2[wid], s + 2);
        issue(ring2[wid], s + 2 + R);
      }
    }
    // every load of this wave has landed before its stages are refilled
    lds_dma_wait<0>();
    __syncthreads();
    if (a.hist) {
      for (int i = 0; i < QR; ++i) {
        if (pos[i] < 0) continue;
        uint32_t* gh = a.hist + ((size_t)b * a.qr + ri0 + i) * NB;
        for (int e = tid; e < NB; e += NT) {
          const uint32_t v = hist[i][e];
          if (v) {
            atomicAdd(&gh[e], v);
            hist[i][e] = 0u;
          }
        }
      }
      __syncthreads();
    }
    while (left > 0 && ++b < a.B && seq_pairs(b) == 0) {
    }
  }
}

}  // namespace pivot
