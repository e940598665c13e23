// FP8-out GEMM, A and B given K-major (layout tag 3); see mm_fp8_km_q8.h.
#include "mm_fp8_km_q8.h"

namespace fp8mi {

hipError_t launch_mm_km_q8_l3(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st) {
  return launch_mm_km_q8_layout<3>(p, fmt_a, fmt_b, st);
}

}  // namespace fp8mi
