// Short-K GEMMs (K <= kPreciseMaxK), bf16 output, K-major operand(s): the
// precise accumulation of mm_fp8_kernel.h with the layout tags.
#include "mm_fp8_kernel.h"

namespace fp8mi {

template <int FA, int FB> static hipError_t launch_prec_km_fmts(const MmArgs& p, hipStream_t st) {
  switch (p.layout) {
    case 1: return launch_dma_precise<FA, FB, -1, 1>(p, st);
    case 2: return launch_dma_precise<FA, FB, -1, 2>(p, st);
    default: return launch_dma_precise<FA, FB, -1, 3>(p, st);
  }
}

hipError_t launch_mm_prec_km(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st) {
  if (fmt_a == kE4M3 && fmt_b == kE4M3) return launch_prec_km_fmts<kE4M3, kE4M3>(p, st);
  if (fmt_a == kE5M2 && fmt_b == kE4M3) return launch_prec_km_fmts<kE5M2, kE4M3>(p, st);
  if (fmt_a == kE4M3 && fmt_b == kE5M2) return launch_prec_km_fmts<kE4M3, kE5M2>(p, st);
  return launch_prec_km_fmts<kE5M2, kE5M2>(p, st);
}

}  // namespace fp8mi
