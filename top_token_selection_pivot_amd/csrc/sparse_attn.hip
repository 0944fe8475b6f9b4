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

// bf16 code of x, round to nearest even (finite inputs)
__device__ inline uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int HB>
__global__ __launch_bounds__(kWave) void sattn_kernel(SAttnArgs a) {
  constexpr int NKS = kAD / 16;   // k-steps of the score contraction
  constexpr int NDB = kADV / 32;  // 32-row blocks of value columns
  __shared__ __attribute__((aligned(16))) uint16_t vs[32][kADV];  // the tile's value rows

  const int lane = threadIdx.x, n = lane & 31, hf = lane >> 5;
  const int r = blockIdx.y, c = blockIdx.x;
  const int s0 = c * a.chunk, s1 = min(s0 + a.chunk, a.nidx);
  const size_t seq = (size_t)(r / a.rows_per_seq);
  const __amdgpu_buffer_rsrc_t kr =
      rsrc(a.k + seq * (size_t)a.seq_stride * kAD, (uint32_t)a.seq_len * kAD * 2u);
  const __amdgpu_buffer_rsrc_t vr =
      rsrc(a.v + seq * (size_t)a.seq_stride * kADV, (uint32_t)a.seq_len * kADV * 2u);
  const int32_t* idx = a.idx + (size_t)r * a.nidx;

  // Q^T as the B operand: lane (head n, half hf) holds q[head][16 ks + 8 hf ..+8]
  i32x4 qf[HB][NKS];
#pragma unroll
  for (int nb = 0; nb < HB; ++nb)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[nb][ks] = *reinterpret_cast<const i32x4*>(a.q + ((size_t)r * a.Hq + nb * 32 + n) * kAD + 16 * ks + 8 * hf);

  f32x16 o[NDB][HB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int nb = 0; nb < HB; ++nb) o[db][nb] = f32x16{};
  float m[HB], l[HB];
#pragma unroll
  for (int nb = 0; nb < HB; ++nb) {
    m[nb] = -INFINITY;
    l[nb] = 0.f;
  }

  // the positions of the next tile are loaded one tile ahead
  int pos_next = s0 + n < s1 ? idx[s0 + n] : -1;
  for (int t0 = s0; t0 < s1; t0 += 32) {
    // this lane's key row (A operand row n) and its validity
    const int pos = pos_next;
    const bool valid = pos >= 0 && pos < a.seq_len;
    const uint32_t vmask = (uint32_t)__ballot(valid);  // bit j: key row j of the tile is valid
    // the tile's value rows go to LDS: piece p = lane + 64 i is 16 bytes of row p / 16
    int rp[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) rp[i] = __shfl(pos, (lane + 64 * i) >> 4);
    // all of the tile's gathers are issued before any of them is used (the
    // compiler would otherwise place each next to its use and wait for it)
    i32x4 kf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kf[ks] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             kr, valid ? (pos * kAD + 16 * ks + 8 * hf) * 2 : 0x80000000u, 0, 0));
    u32x4 vv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = lane + 64 * i, row = p >> 4, ch = p & 15;
      const bool rv = (vmask >> row) & 1u;
      vv[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, rv ? (rp[i] * kADV + 8 * ch) * 2 : 0x80000000u, 0, 0);
    }
    pos_next = t0 + 32 + n < s1 ? idx[t0 + 32 + n] : -1;
    __builtin_amdgcn_sched_barrier(0);
    // scores S^T (32 keys x 32 heads per head block)
    f32x16 s[HB];
#pragma unroll
    for (int nb = 0; nb < HB; ++nb) {
      s[nb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        s[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[ks]),
                                                        __builtin_bit_cast(bf16x8, qf[nb][ks]), s[nb], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = lane + 64 * i;
      *reinterpret_cast<u32x4*>(&vs[p >> 4][8 * (p & 15)]) = vv[i];
    }
    // online softmax of head n (block nb): accumulator i holds key row
    // 8 (i / 4) + 4 hf + i % 4 of the tile
    i32x4 phi[HB][2], plo[HB][2];
#pragma unroll
    for (int nb = 0; nb < HB; ++nb) {
      float x[16];
      float mt = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * hf + (i & 3);
        x[i] = ((vmask >> key) & 1u) ? s[nb][i] * a.scale : -INFINITY;
        mt = fmaxf(mt, x[i]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m[nb], mt);
      const float base = mn == -INFINITY ? 0.f : mn;
      const float alpha = __expf(m[nb] - base);  // 0 while nothing was seen
      float ls = 0.f;
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = __expf(x[i] - base);
        ls += p[i];
      }
      ls += __shfl_xor(ls, 32);
      l[nb] = l[nb] * alpha + ls;
      m[nb] = mn;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][nb][i] *= alpha;
      // P as the B operand of k-step ks2: elements j = 0..7 are accumulators 8 ks2 + j
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float a0 = p[8 * ks2 + 2 * w], a1 = p[8 * ks2 + 2 * w + 1];
          const uint32_t h0 = bf16_rne(a0), h1 = bf16_rne(a1);
          const uint32_t l0 = bf16_rne(a0 - __uint_as_float(h0 << 16));
          const uint32_t l1 = bf16_rne(a1 - __uint_as_float(h1 << 16));
          phi[nb][ks2][w] = (int)(h0 | (h1 << 16));
          plo[nb][ks2][w] = (int)(l0 | (l1 << 16));
        }
    }
    // value tile written by every lane before it is read
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O^T += V^T P: A fragment of k-step ks2 for value column 32 db + n holds the
    // values of keys 16 ks2 + 8 (j / 4) + 4 hf + j % 4, j = 0..7
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const int k0 = 16 * ks2 + 4 * hf, col = 32 * db + n;
        i32x4 af;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int j0 = 2 * w, j1 = 2 * w + 1;
          const uint32_t e0 = vs[k0 + 8 * (j0 >> 2) + (j0 & 3)][col];
          const uint32_t e1 = vs[k0 + 8 * (j1 >> 2) + (j1 & 3)][col];
          af[w] = (int)(e0 | (e1 << 16));
        }
#pragma unroll
        for (int nb = 0; nb < HB; ++nb) {
          o[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af),
                                                              __builtin_bit_cast(bf16x8, phi[nb][ks2]), o[db][nb], 0, 0, 0);
          o[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af),
                                                              __builtin_bit_cast(bf16x8, plo[nb][ks2]), o[db][nb], 0, 0, 0);
        }
      }
    // every lane has read the value tile before the next one is written
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
  }

  // lane (head n, half hf) holds value columns 32 db + 8 (i / 4) + 4 hf + i % 4
#pragma unroll
  for (int nb = 0; nb < HB; ++nb) {
    const int head = nb * 32 + n;
    if (a.nch == 1) {
      const float inv = l[nb] > 0.f ? 1.f / l[nb] : 0.f;
      float* dst = a.out + ((size_t)r * a.Hq + head) * kADV;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = 32 * db + 8 * g4 + 4 * hf;
          *reinterpret_cast<float4*>(dst + col) =
              make_float4(o[db][nb][4 * g4] * inv, o[db][nb][4 * g4 + 1] * inv, o[db][nb][4 * g4 + 2] * inv,
                          o[db][nb][4 * g4 + 3] * inv);
        }
    } else {
      const size_t pc = (size_t)r * a.nch + c;
      float* dst = a.part_o + (pc * a.Hq + head) * kADV;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = 32 * db + 8 * g4 + 4 * hf;
          *reinterpret_cast<float4*>(dst + col) =
              make_float4(o[db][nb][4 * g4], o[db][nb][4 * g4 + 1], o[db][nb][4 * g4 + 2], o[db][nb][4 * g4 + 3]);
        }
      if (hf == 0) {
        a.part_ml[pc * 2 * a.Hq + head] = m[nb];
        a.part_ml[pc * 2 * a.Hq + a.Hq + head] = l[nb];
      }
    }
  }
}

// Merges the chunks of one (row, head): with M the largest chunk maximum,
// out = sum_c exp(m_c - M) o_c / sum_c exp(m_c - M) l_c (zeros when the row
// selected nothing).  One thread per value column; the chunk loop is unrolled
// so that the chunks' loads are in flight together.
__global__ __launch_bounds__(kADV) void sattn_combine_kernel(SAttnArgs a) {
  const int r = blockIdx.y, h = blockIdx.x, col = threadIdx.x;
  const size_t p0 = (size_t)r * a.nch;
  float M = -INFINITY;
  for (int c = 0; c < a.nch; ++c) M = fmaxf(M, a.part_ml[(p0 + c) * 2 * a.Hq + h]);
  float acc = 0.f, L = 0.f;
  if (M != -INFINITY) {
#pragma unroll 8
    for (int c = 0; c < a.nch; ++c) {
      const float* ml = a.part_ml + (p0 + c) * 2 * a.Hq;
      const float wgt = __expf(ml[h] - M);
      L += wgt * ml[a.Hq + h];
      acc += wgt * a.part_o[((p0 + c) * a.Hq + h) * kADV + col];
    }
  }
  a.out[((size_t)r * a.Hq + h) * kADV + col] = L > 0.f ? acc / L : 0.f;
}

}  // namespace

bool sattn_shape_supported(int Hq, int d, int dv) { return d == kAD && dv == kADV && (Hq == 32 || Hq == 64); }

hipError_t launch_sparse_attention(const SAttnArgs& a, hipStream_t st) {
  if (a.R <= 0) return hipSuccess;
  dim3 grid(a.nch, a.R);
  if (a.Hq == 32)
    hipLaunchKernelGGL(sattn_kernel<1>, grid, dim3(kWave), 0, st, a);
  else
    hipLaunchKernelGGL(sattn_kernel<2>, grid, dim3(kWave), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nch == 1) return e;
  hipLaunchKernelGGL(sattn_combine_kernel, dim3(a.Hq, a.R), dim3(kADV), 0, st, a);
  return hipGetLastError();
}

}  // namespace pivot
