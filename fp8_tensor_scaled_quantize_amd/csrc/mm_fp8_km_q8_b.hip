// FP8-out GEMM, B given K-major (layout tag 2); see mm_fp8_km_q8.h.
#include "mm_fp8_km_q8.h"

namespace fp8mi {

hipError_t launch_mm_km_q8_l2(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st) {
  return launch_mm_km_q8_layout<2>(p, fmt_a, fmt_b, st);
}

}  // namespace fp8mi
