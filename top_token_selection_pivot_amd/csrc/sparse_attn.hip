// sparse_attn.hip -- sparse main attention over the selected positions (gfx950).
//
// Tutorial "Sparse Attention의 Indexer", text after Figure 1: the main query
// scores the main keys at the positions the indexer selected, and the values
// there are combined with softmax weights over those positions only.  Layout:
// one key row and one value row per position, shared by the query heads
// (multi-query), bf16 codes, head dimensions D = DV = 128, 32 or 64 heads.
//
// One wave takes one query row and a chunk of its selected slots, 32 at a time:
//   S^T = K_sel . Q^T on the matrix cores (keys on M: every lane loads its key
//     row's slice of the A fragment straight from memory; heads on N: the
//     query stays in registers), so lane (head n, half hf) holds the scores of
//     head n for 16 of the 32 keys and the online softmax of head n is in-lane
//     plus one exchange with the other half;
//   O^T += V^T . P on the matrix cores: P is the B operand as it sits in the
//     score accumulators (keys in the order the accumulator rows give, which
//     the A fragments of V^T, read from the value tile in LDS, follow too);
//     P is split into two bf16 terms (P = hi + lo), which keeps its rounding
//     error near 2^-17 instead of 2^-9.
// A row's slots form one chunk when there are many rows; otherwise every
// chunk writes its unnormalised output, running maximum and sum, and a second
// kernel merges the chunks.
// ---------------------------------------------------------------------------
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pivot_device.h"
#include "pivot_kernels.h"

namespace pivot {
namespace {

constexpr int kAD = 128;   // key / query head dimension
constexpr int kADV = 128;  // value head dimension
constexpr uint32_t kRangeFlags = 0x00020000;  // raw 32-bit buffer, range-checked

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRangeFlags);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// two floats as packed bf16 codes, round to nearest even (one conversion instruction)
__device__ inline uint32_t bf16x2_rne(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){x0, x1}, bf16x2_t));
}

// The softmax runs in base-2 units: a score is scaled once by scale * log2(e),
// so every weight is one exp2 of a difference (exp(scale*x - c) = 2^(x' - c')).
// The running maximum of a head moves only when a tile's maximum exceeds it by
// more than kLazyMax (base-2 units), so the output is rarely rescaled; the
// weights 2^(x - m) then stay below 2^kLazyMax.  The result is the same in
// exact arithmetic: the output and the sum always refer to the same m.
constexpr float kLazyMax = 12.f;
constexpr float kLog2e = 1.4426950408889634f;
__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// A workgroup holds NW = Hq / 32 waves on the same (chunk, row); wave w takes
// heads 32 w .. 32 w + 31.  With 64 heads a wave keeps its registers under
// 256, so two waves share a SIMD and one's memory waits overlap the other's
// work (a 32-head wave gathers alone and holds twice the pieces).  The
// workgroup gathers each tile's key and value rows once, whole 256-byte rows
// split over its waves, into LDS (double buffered, 16-byte chunks of row j
// XOR-swizzled by j % 16 so that the fragment reads of 32 rows spread over
// the banks); the next tile's rows are in flight in registers while the
// current tile is computed, and one barrier per tile hands a tile over.
template <int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(NW))) void sattn_kernel(SAttnArgs a) {
  constexpr int NKS = kAD / 16;   // k-steps of the score contraction
  constexpr int NDB = kADV / 32;  // 32-row blocks of value columns
  constexpr int ROWB = kAD * 2;   // bytes of a key row (= a value row)
  constexpr int TILE = 32 * ROWB;
  constexpr int PPL = 32 * (ROWB / 16) / (NW * kWave);  // 16-byte pieces per lane per tile and matrix
  static_assert(kAD == kADV && PPL * NW * kWave == 32 * (ROWB / 16));
  __shared__ __attribute__((aligned(16))) uint8_t kt[2][TILE];
  __shared__ __attribute__((aligned(16))) uint8_t vt[2][TILE];

  const int tid = threadIdx.x, lane = tid & 63, n = lane & 31, hf = lane >> 5;
  const int hb = __builtin_amdgcn_readfirstlane(tid >> 6);  // head block of this wave
  const int r = blockIdx.y, c = blockIdx.x;
  const int s0 = c * a.chunk, s1 = min(s0 + a.chunk, a.nidx);
  const size_t seq = (size_t)(r / a.rows_per_seq);
  const __amdgpu_buffer_rsrc_t kr =
      rsrc(a.k + seq * (size_t)a.seq_stride * kAD, (uint32_t)a.seq_len * kAD * 2u);
  const __amdgpu_buffer_rsrc_t vr =
      rsrc(a.v + seq * (size_t)a.seq_stride * kADV, (uint32_t)a.seq_len * kADV * 2u);
  const int32_t* idx = a.idx + (size_t)r * a.nidx;
  const int head = hb * 32 + n;
  // byte offset of 16-byte chunk ch of row j in a tile
  auto chunk_at = [](int j, int ch) { return j * ROWB + ((ch ^ (j & 15)) << 4); };
  // this lane's row and column within a half k-step of the value tile for
  // the transposing reads of V^T (see below)
  const int tr_row = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // Q^T as the B operand: lane (head n, half hf) holds q[head][16 ks + 8 hf ..+8]
  i32x4 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    qf[ks] = *reinterpret_cast<const i32x4*>(a.q + ((size_t)r * a.Hq + head) * kAD + 16 * ks + 8 * hf);

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m = -INFINITY, l = 0.f;  // running maximum (base-2 units) and sum
  const float sl2 = a.scale * kLog2e;

  // lane n (and n + 32) holds the position of slot n of the tile at t0
  auto load_pos = [&](int t0) { return t0 + n < s1 ? idx[t0 + n] : -1; };
  // piece p = tid + NW * 64 * i of a tile is chunk p % 16 of row p / 16
  i32x4 gk[PPL], gv[PPL];
  auto gather = [&](int posv) {
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
      const int p = tid + NW * kWave * i, j = p >> 4, ch = p & 15;
      const int ps = __shfl(posv, j);
      const bool ok = ps >= 0 && ps < a.seq_len;
      gk[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            kr, ok ? (ps * kAD + 8 * ch) * 2 : 0x80000000u, 0, 0));
      gv[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            vr, ok ? (ps * kADV + 8 * ch) * 2 : 0x80000000u, 0, 0));
    }
  };
  auto stash = [&](int b) {
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
      const int p = tid + NW * kWave * i, j = p >> 4, ch = p & 15;
      *reinterpret_cast<i32x4*>(&kt[b][chunk_at(j, ch)]) = gk[i];
      *reinterpret_cast<i32x4*>(&vt[b][chunk_at(j, ch)]) = gv[i];
    }
  };

  auto compute = [&](int b, int posv) {
    const bool valid = posv >= 0 && posv < a.seq_len;
    const uint32_t vmask = (uint32_t)__ballot(valid);  // bit j: key row j of the tile is valid
    // scores S^T (32 keys x 32 heads): A fragment = elements 16 ks + 8 hf ..+8 of key row n
    f32x16 sc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const i32x4 kf = *reinterpret_cast<const i32x4*>(&kt[b][chunk_at(n, 2 * ks + hf)]);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf),
                                                   __builtin_bit_cast(bf16x8, qf[ks]), sc, 0, 0, 0);
    }
    // online softmax of head n: accumulator i holds key row 8 (i / 4) + 4 hf + i % 4
    float mt = -INFINITY;
    if (vmask == 0xFFFFFFFFu) {  // the usual tile: every key valid
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[i] *= sl2;
        mt = fmaxf(mt, sc[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * hf + (i & 3);
        sc[i] = ((vmask >> key) & 1u) ? sc[i] * sl2 : -INFINITY;
        mt = fmaxf(mt, sc[i]);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool grow = mt > m + kLazyMax;  // with m = -inf: any valid key
    const float mn = grow ? mt : m;
    const float alpha = grow ? exp2_fast(m - mn) : 1.f;  // 0 on the first tile with a valid key
    const float base = mn == -INFINITY ? 0.f : mn;
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sc[i] = exp2_fast(sc[i] - base);
      ls += sc[i];
    }
    ls += __shfl_xor(ls, 32);
    l = l * alpha + ls;
    // the output is zero until a head's first valid key, so only a lane whose
    // maximum moved after that needs the rescale
    if (__ballot(grow && m != -INFINITY)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    m = mn;
    // P as the B operand of k-step ks2: elements j = 0..7 are accumulators 8 ks2 + j
    i32x4 phi[2], plo[2];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a0 = sc[8 * ks2 + 2 * w], a1 = sc[8 * ks2 + 2 * w + 1];
        const uint32_t h = bf16x2_rne(a0, a1);
        phi[ks2][w] = (int)h;
        plo[ks2][w] = (int)bf16x2_rne(a0 - __uint_as_float(h << 16), a1 - __uint_as_float(h & 0xFFFF0000u));
      }
    // O^T += V^T P: A fragment of k-step ks2 for value column 32 db + n holds the
    // values of keys 16 ks2 + 8 (j / 4) + 4 hf + j % 4, j = 0..7.  Each half
    // (j = 0..3, j = 4..7) is one transposing LDS read: in every group of 16
    // lanes, lane i names 4 consecutive values M_i[0..3] of a value row and
    // lane j receives M_{4e + j/4}[j % 4], e = 0..3; so lane 16 G + i names
    // row 4 (G / 2) + i / 4 of the half, columns 16 (G % 2) + 4 (i % 4) ..+3.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const int j0 = 16 * ks2 + tr_row, j1 = j0 + 8, col = 32 * db + tr_col;
        const v4i16 e0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)&vt[b][chunk_at(j0, col >> 3) + (col & 7) * 2]);
        const v4i16 e1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)&vt[b][chunk_at(j1, col >> 3) + (col & 7) * 2]);
        const i32x4 af = __builtin_bit_cast(i32x4, (v8i16){e0[0], e0[1], e0[2], e0[3], e1[0], e1[1], e1[2], e1[3]});
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af),
                                                        __builtin_bit_cast(bf16x8, phi[ks2]), o[db], 0, 0, 0);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af),
                                                        __builtin_bit_cast(bf16x8, plo[ks2]), o[db], 0, 0, 0);
      }
  };

  // tile k's rows sit in buffer k % 2; tile k + 1's are in flight meanwhile
  int pc = load_pos(s0), pn = load_pos(s0 + 32);
  gather(pc);
  stash(0);
  gather(pn);
  __syncthreads();
  int b = 0;
  for (int t0 = s0; t0 < s1; t0 += 32) {
    const int pnn = load_pos(t0 + 64);
    compute(b, pc);
    stash(b ^ 1);  // every wave is done with that buffer since the last barrier
    gather(pnn);
    __syncthreads();
    pc = pn;
    pn = pnn;
    b ^= 1;
  }

  // lane (head n, half hf) holds value columns 32 db + 8 (i / 4) + 4 hf + i % 4
  if (a.nch == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* dst = a.out + ((size_t)r * a.Hq + head) * kADV;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int col = 32 * db + 8 * g4 + 4 * hf;
        *reinterpret_cast<float4*>(dst + col) = make_float4(o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv,
                                                            o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv);
      }
  } else {
    const size_t pc2 = (size_t)r * a.nch + c;
    float* dst = a.part_o + (pc2 * a.Hq + head) * kADV;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int col = 32 * db + 8 * g4 + 4 * hf;
        *reinterpret_cast<float4*>(dst + col) =
            make_float4(o[db][4 * g4], o[db][4 * g4 + 1], o[db][4 * g4 + 2], o[db][4 * g4 + 3]);
      }
    if (hf == 0) {
      a.part_ml[pc2 * 2 * a.Hq + head] = m;
      a.part_ml[pc2 * 2 * a.Hq + a.Hq + head] = l;
    }
  }
}

// Merges the chunks of one (row, head): with M the largest chunk maximum
// (base-2 units, as the chunks store them),
// out = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c (zeros when the row
// selected nothing).  A thread takes four value columns of one (row, head) and
// up to kMergeChunks chunks at a time: every chunk's maximum, sum and partial
// output are loaded before any is used (indices clamped, so no load is
// conditional), which leaves one memory latency per round; a later round
// rescales what the earlier ones accumulated.
constexpr int kMergeChunks = 16;
constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void sattn_combine_kernel(SAttnArgs a) {
  const long long t = (long long)blockIdx.x * kMergeThreads + threadIdx.x;
  const int q4 = (int)(t & 31);  // columns 4 q4 .. 4 q4 + 3
  const long long rh = t >> 5;   // r * Hq + h
  if (rh >= (long long)a.R * a.Hq) return;
  const int r = (int)(rh / a.Hq), h = (int)(rh % a.Hq);
  const size_t p0 = (size_t)r * a.nch;
  float M = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < a.nch; c0 += kMergeChunks) {
    float mc[kMergeChunks], lc[kMergeChunks];
    float4 oc[kMergeChunks];
#pragma unroll
    for (int i = 0; i < kMergeChunks; ++i) {
      const size_t pc = p0 + min(c0 + i, a.nch - 1);
      mc[i] = a.part_ml[pc * 2 * a.Hq + h];
      lc[i] = a.part_ml[pc * 2 * a.Hq + a.Hq + h];
      oc[i] = *reinterpret_cast<const float4*>(a.part_o + (pc * a.Hq + h) * kADV + 4 * q4);
    }
    float Mn = M;
#pragma unroll
    for (int i = 0; i < kMergeChunks; ++i) {
      if (c0 + i >= a.nch) mc[i] = -INFINITY;  // a clamped duplicate
      Mn = fmaxf(Mn, mc[i]);
    }
    if (Mn == -INFINITY) continue;  // nothing selected so far
    const float sc = exp2_fast(M - Mn);  // 0 on the first round that sees a slot
    L *= sc;
    acc.x *= sc;
    acc.y *= sc;
    acc.z *= sc;
    acc.w *= sc;
#pragma unroll
    for (int i = 0; i < kMergeChunks; ++i) {
      const float wgt = exp2_fast(mc[i] - Mn);
      L += wgt * lc[i];
      acc.x += wgt * oc[i].x;
      acc.y += wgt * oc[i].y;
      acc.z += wgt * oc[i].z;
      acc.w += wgt * oc[i].w;
    }
    M = Mn;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<float4*>(a.out + rh * kADV + 4 * q4) =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

}  // namespace

bool sattn_shape_supported(int Hq, int d, int dv) { return d == kAD && dv == kADV && (Hq == 32 || Hq == 64); }

hipError_t launch_sparse_attention(const SAttnArgs& a, hipStream_t st) {
  if (a.R <= 0) return hipSuccess;
  dim3 grid(a.nch, a.R);
  if (a.Hq == 32)
    hipLaunchKernelGGL(sattn_kernel<1>, grid, dim3(kWave), 0, st, a);
  else
    hipLaunchKernelGGL(sattn_kernel<2>, grid, dim3(2 * kWave), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nch == 1) return e;
  const long long threads = (long long)a.R * a.Hq * (kADV / 4);
  hipLaunchKernelGGL(sattn_combine_kernel, dim3((unsigned)((threads + kMergeThreads - 1) / kMergeThreads)),
                     dim3(kMergeThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace pivot
