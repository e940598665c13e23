// Short-K GEMMs (K <= kPreciseMaxK) with the quantizing (fp8-out) epilogue:
// the precise accumulation of mm_fp8_kernel.h; empty outputs and the zeroed
// amax word are handled by the caller (launch_mm_q8) as for every K.
#include "mm_fp8_kernel.h"

namespace fp8mi {

template <int FA, int FB> static hipError_t launch_prec_out(const MmArgs& p, hipStream_t st) {
  return p.out_fmt == kE4M3 ? launch_dma_precise<FA, FB, kE4M3, 0>(p, st)
                            : launch_dma_precise<FA, FB, kE5M2, 0>(p, st);
}

hipError_t launch_mm_prec_q8(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st) {
  if (fmt_a == kE4M3 && fmt_b == kE4M3) return launch_prec_out<kE4M3, kE4M3>(p, st);
  if (fmt_a == kE5M2 && fmt_b == kE4M3) return launch_prec_out<kE5M2, kE4M3>(p, st);
  if (fmt_a == kE4M3 && fmt_b == kE5M2) return launch_prec_out<kE4M3, kE5M2>(p, st);
  return launch_prec_out<kE5M2, kE5M2>(p, st);
}

}  // namespace fp8mi
