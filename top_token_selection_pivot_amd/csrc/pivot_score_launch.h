// pivot_score_launch.h -- shape dispatch of the scoring kernels for one code
// type; included once per code type so the two compile in parallel.
#pragma once

#include "pivot_score.h"

namespace pivot {

// Compute units of the current device.
static inline int device_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || cus < 1)
    cus = 1;
  return cus;
}

template <int DT, int D, int HB>
static void scan_one(const ScanArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((score_block_kernel<DT, D, HB, false, kScanRows, ScanArgs>), grid, dim3(kScanRows * kWave), 0,
                     st, a);
}
// Refine workgroups have as many waves as a group has members (2, 4 or 8).
template <int DT, int D, int HB>
static void refine_one(const RefineArgs& a, dim3 grid, int rows, hipStream_t st) {
  if (rows == 2)
    hipLaunchKernelGGL((score_block_kernel<DT, D, HB, true, 2, RefineArgs>), grid, dim3(2 * kWave), 0, st, a);
  else if (rows == 4)
    hipLaunchKernelGGL((score_block_kernel<DT, D, HB, true, 4, RefineArgs>), grid, dim3(4 * kWave), 0, st, a);
  else
    hipLaunchKernelGGL((score_block_kernel<DT, D, HB, true, 8, RefineArgs>), grid, dim3(8 * kWave), 0, st, a);
}
// Decode scan workgroups are persistent: as many as fit on the chip at once.
template <int DT, int D, int HB, int QR, bool PAGED>
static void decode_launch(const DecScanArgs& a, int zblocks, hipStream_t st) {
  using G = DecGeom<DT, D, QR>;
  static const int per_cu = [] {
    int nblk = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nblk, decode_scan_kernel<DT, D, HB, QR, PAGED>, G::THREADS,
                                                     0) != hipSuccess ||
        nblk < 1)
      nblk = 1;
    return nblk;
  }();
  dim3 grid(device_cu_count() * per_cu, 1, zblocks);
  hipLaunchKernelGGL((decode_scan_kernel<DT, D, HB, QR, PAGED>), grid, dim3(G::THREADS), 0, st, a);
}
template <int DT, int D, int HB, bool PAGED>
static void decode_qr(const DecScanArgs& a, int zblocks, hipStream_t st) {
  if (a.qr == 1)
    decode_launch<DT, D, HB, 1, PAGED>(a, zblocks, st);
  else
    decode_launch<DT, D, HB, 2, PAGED>(a, zblocks, st);
}
template <int DT, int D, int HB>
static void decode_one(const DecScanArgs& a, int zblocks, hipStream_t st) {
  if (a.bt)
    decode_qr<DT, D, HB, true>(a, zblocks, st);
  else
    decode_qr<DT, D, HB, false>(a, zblocks, st);
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

constexpr int kScanMaxKeyChunk = 16384;

// Keys per scan workgroup: a.kc at least, and as long as keeps about 8
// workgroups per compute unit over this launch's causal triangle (each
// workgroup first loads its 8 query rows and first key stage, so longer
// chunks amortise that), at most kScanMaxKeyChunk.
static inline int scan_key_chunk(const ScanArgs& a) {
  long long total = 0;
  for (int rb = a.row_begin; rb < a.row_end; rb += kScanRows) {
    const int rl = min(rb + kScanRows, a.row_end) - 1;
    total += min(rl * a.pos_mul + a.pos_add, a.pos_cap) + 1;
  }
  long long kc = total / (8LL * device_cu_count());
  kc = (kc + 255) / 256 * 256;
  return (int)std::max<long long>(a.kc, std::min<long long>(kc, kScanMaxKeyChunk));
}

template <int DT>
hipError_t launch_scan_dt(const ScanArgs& a_in, int D, hipStream_t st) {
  ScanArgs a = a_in;
  a.kc = scan_key_chunk(a_in);
  const int nrows = a.row_end - a.row_begin;
  const int rlast = a.row_end - 1;
  const int lim = min(rlast * a.pos_mul + a.pos_add, a.pos_cap) + 1;
  if (nrows <= 0 || lim <= 0) return hipSuccess;  // no row sees any key
  a.nchunks = (lim + a.kc - 1) / a.kc;
  a.nblocks = (nrows + kScanRows - 1) / kScanRows;
  const long long n = (long long)a.nchunks * a.nblocks;
  dim3 grid((unsigned)((n + 7) / 8 * 8));  // a multiple of the eight XCDs
  auto f = [&]<int D_, int HB_>() { scan_one<DT, D_, HB_>(a, grid, st); };
  if (!dispatch_shape<DT>(D, a.H, f)) return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int DT>
hipError_t launch_refine_dt(const RefineArgs& a_in, int D, hipStream_t st) {
  RefineArgs a = a_in;
  const int ngrp = a.grp_end - a.grp_begin;
  const int rows = a.g <= 2 ? 2 : a.g <= 4 ? 4 : kScanRows;
  const int zblocks = (a.g + rows - 1) / rows;
  // all candidates in one workgroup when there are enough groups to fill the
  // chip (each member's query is then loaded once); otherwise the candidates
  // are split into as few pieces (of at least 256 slots) as bring the launch
  // to about 2048 workgroups
  const long long units = (long long)ngrp * zblocks;
  const int full = min(a.m, kRefineSlotMax);
  if (units >= 2048) {
    a.slot_chunk = full;
  } else {
    const long long parts = (2048 + units - 1) / units;
    a.slot_chunk = (int)std::max<long long>(256, ((full + parts - 1) / parts + 255) / 256 * 256);
  }
  dim3 grid((a.m + a.slot_chunk - 1) / a.slot_chunk, ngrp, zblocks);
  auto f = [&]<int D_, int HB_>() { refine_one<DT, D_, HB_>(a, grid, rows, st); };
  if (!dispatch_shape<DT>(D, a.H, f)) return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int DT>
hipError_t launch_decode_scan_dt(const DecScanArgs& a, int D, hipStream_t st) {
  const int zblocks = a.qr == 1 ? 1 : (a.qr + 1) / 2;
  auto f = [&]<int D_, int HB_>() { decode_one<DT, D_, HB_>(a, zblocks, st); };
  if (!dispatch_shape<DT>(D, a.H, f)) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pivot
