// FP8-out GEMM, A given K-major (layout tag 1); see mm_fp8_km_q8.h.
#include "mm_fp8_km_q8.h"

namespace fp8mi {

hipError_t launch_mm_km_q8_l1(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st) {
  return launch_mm_km_q8_layout<1>(p, fmt_a, fmt_b, st);
}

}  // namespace fp8mi
