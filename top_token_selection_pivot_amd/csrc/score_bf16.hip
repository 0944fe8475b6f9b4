// score_bf16.hip -- bf16 instantiations of the scoring kernels.
#include "pivot_score_launch.h"

namespace pivot {
hipError_t launch_scan_bf16(const ScanArgs& a, int D, hipStream_t st) {
  return launch_scan_dt<kBF16>(a, D, st);
}
hipError_t launch_refine_bf16(const RefineArgs& a, int D, hipStream_t st) {
  return launch_refine_dt<kBF16>(a, D, st);
}
hipError_t launch_decode_scan_bf16(const DecScanArgs& a, int D, hipStream_t st) {
  return launch_decode_scan_dt<kBF16>(a, D, st);
}
}  // namespace pivot
