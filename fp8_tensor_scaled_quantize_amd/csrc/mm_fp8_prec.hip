// Short-K GEMMs (K <= kPreciseMaxK), bf16 output, NT operands: the mm_fp8_dma
// kernels with the precise accumulation (one product per MFMA group of 8 k,
// mm_fp8_kernel.h), so that the fp8 MFMA's in-group truncation stays out of
// the result where 1e-5 * sum |a b| leaves it least room.
#include "mm_fp8_kernel.h"

namespace fp8mi {

hipError_t launch_mm_prec_nt(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st) {
  if (fmt_a == kE4M3 && fmt_b == kE4M3) return launch_dma_precise<kE4M3, kE4M3, -1, 0>(p, st);
  if (fmt_a == kE5M2 && fmt_b == kE4M3) return launch_dma_precise<kE5M2, kE4M3, -1, 0>(p, st);
  if (fmt_a == kE4M3 && fmt_b == kE5M2) return launch_dma_precise<kE4M3, kE5M2, -1, 0>(p, st);
  return launch_dma_precise<kE5M2, kE5M2, -1, 0>(p, st);
}

}  // namespace fp8mi
