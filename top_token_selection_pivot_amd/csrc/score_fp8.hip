// score_fp8.hip -- OCP FP8 E4M3 instantiations of the scoring kernels.
#include "pivot_score_launch.h"

namespace pivot {
hipError_t launch_scan_fp8(const ScanArgs& a, int D, hipStream_t st) {
  return launch_scan_dt<kFP8>(a, D, st);
}
hipError_t launch_refine_fp8(const RefineArgs& a, int D, hipStream_t st) {
  return launch_refine_dt<kFP8>(a, D, st);
}
hipError_t launch_decode_scan_fp8(const DecScanArgs& a, int D, hipStream_t st) {
  return launch_decode_scan_dt<kFP8>(a, D, st);
}
}  // namespace pivot
