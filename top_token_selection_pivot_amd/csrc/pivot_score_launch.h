// pivot_score_launch.h -- shape dispatch of the scoring kernels for one code
// type; included once per code type so the two compile in parallel.
#pragma once

#include "pivot_score.h"

namespace pivot {

template <int DT, int D, int HB>
static void scan_one(const ScanArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((score_block_kernel<DT, D, HB, false, ScanArgs>), grid, dim3(kScanWaveThreads), 0, st, a);
}
template <int DT, int D, int HB>
static void refine_one(const RefineArgs& a, dim3 grid, dim3 block, hipStream_t st) {
  hipLaunchKernelGGL((score_block_kernel<DT, D, HB, true, RefineArgs>), grid, dim3(kScanWaveThreads), 0, st, a);
}
template <int DT, int D, int HB>
static void decode_one(const DecScanArgs& a, dim3 grid, hipStream_t st) {
  if (a.qr == 1)
    hipLaunchKernelGGL((decode_scan_kernel<DT, D, HB, 1>), grid, dim3(kDecThreads), 0, st, a);
  else
    hipLaunchKernelGGL((decode_scan_kernel<DT, D, HB, 2>), grid, dim3(kDecThreads), 0, st, a);
}

// Calls f.operator()<D, HB>() for the supported head-dimension / head-block combination.
template <int DT, typename F>
static bool dispatch_shape(int D, int H, F&& f) {
  const bool two = H > 32;
  if constexpr (DT == kBF16) {
    switch (D) {
      case 32: two ? f.template operator()<32, 2>() : f.template operator()<32, 1>(); return true;
      case 64: two ? f.template operator()<64, 2>() : f.template operator()<64, 1>(); return true;
      case 128: two ? f.template operator()<128, 2>() : f.template operator()<128, 1>(); return true;
      case 256: two ? f.template operator()<256, 2>() : f.template operator()<256, 1>(); return true;
    }
  } else {
    switch (D) {
      case 64: two ? f.template operator()<64, 2>() : f.template operator()<64, 1>(); return true;
      case 128: two ? f.template operator()<128, 2>() : f.template operator()<128, 1>(); return true;
      case 256: two ? f.template operator()<256, 2>() : f.template operator()<256, 1>(); return true;
    }
  }
  return false;
}

template <int DT>
hipError_t launch_scan_dt(const ScanArgs& a, int D, hipStream_t st) {
  const int nrows = a.row_end - a.row_begin;
  const int rlast = a.row_end - 1;
  const int lim = min(rlast * a.pos_mul + a.pos_add, a.pos_cap) + 1;
  dim3 grid((lim + a.kc - 1) / a.kc, (nrows + kScanRows - 1) / kScanRows);
  auto f = [&]<int D_, int HB_>() { scan_one<DT, D_, HB_>(a, grid, st); };
  if (!dispatch_shape<DT>(D, a.H, f)) return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int DT>
hipError_t launch_refine_dt(const RefineArgs& a, int D, hipStream_t st) {
  const int ngrp = a.grp_end - a.grp_begin;
  dim3 grid((a.m + a.slot_chunk - 1) / a.slot_chunk, ngrp, (a.g + kScanRows - 1) / kScanRows);
  dim3 block(kScanWaveThreads);
  auto f = [&]<int D_, int HB_>() { refine_one<DT, D_, HB_>(a, grid, block, st); };
  if (!dispatch_shape<DT>(D, a.H, f)) return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int DT>
hipError_t launch_decode_scan_dt(const DecScanArgs& a, int D, int B, hipStream_t st) {
  const int qr_step = a.qr == 1 ? 1 : 2;
  dim3 grid((a.Lmax + a.kc - 1) / a.kc, B, (a.qr + qr_step - 1) / qr_step);
  auto f = [&]<int D_, int HB_>() { decode_one<DT, D_, HB_>(a, grid, st); };
  if (!dispatch_shape<DT>(D, a.H, f)) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pivot
