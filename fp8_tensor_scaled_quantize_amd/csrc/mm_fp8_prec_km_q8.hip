// Short-K GEMMs (K <= kPreciseMaxK) with the quantizing (fp8-out) epilogue
// and K-major operand(s): the precise accumulation of mm_fp8_kernel.h with
// the layout tags; empty outputs and the zeroed amax word are handled by the
// caller (launch_mm_q8) as for every K.
#include "mm_fp8_kernel.h"

namespace fp8mi {

template <int FA, int FB, int OUT> static hipError_t prec_km_q8_layout(const MmArgs& p, hipStream_t st) {
  switch (p.layout) {
    case 1: return launch_dma_precise<FA, FB, OUT, 1>(p, st);
    case 2: return launch_dma_precise<FA, FB, OUT, 2>(p, st);
    default: return launch_dma_precise<FA, FB, OUT, 3>(p, st);
  }
}

template <int FA, int FB> static hipError_t prec_km_q8_out(const MmArgs& p, hipStream_t st) {
  return p.out_fmt == kE4M3 ? prec_km_q8_layout<FA, FB, kE4M3>(p, st) : prec_km_q8_layout<FA, FB, kE5M2>(p, st);
}

hipError_t launch_mm_prec_km_q8(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st) {
  if (fmt_a == kE4M3 && fmt_b == kE4M3) return prec_km_q8_out<kE4M3, kE4M3>(p, st);
  if (fmt_a == kE5M2 && fmt_b == kE4M3) return prec_km_q8_out<kE5M2, kE4M3>(p, st);
  if (fmt_a == kE4M3 && fmt_b == kE5M2) return prec_km_q8_out<kE4M3, kE5M2>(p, st);
  return prec_km_q8_out<kE5M2, kE5M2>(p, st);
}

}  // namespace fp8mi
