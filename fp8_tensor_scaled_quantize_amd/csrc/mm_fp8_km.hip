// GEMM with layout tags: A and / or B given K-major ([K, M] / [K, N], the
// layout of a transposed view), read without a transposed copy (the pages'
// layout tags from .t() views: log:tests/extension, the commit taking 3-D and
// transposed operands into the GEMM).  The mm_fp8_dma kernels load such a
// tile into LDS as k-rows (LDS-DMA, swizzled 16-byte chunks) and build the
// MFMA operand fragments with gfx950's LDS transpose read (ds_read_b64_tr_b8).
// bf16 output (fp8 output: mm_fp8_km_q8.h); the same tile family and
// dispatch as the NT GEMM (64 x 64 included).
#include "mm_fp8_kernel.h"

namespace fp8mi {

template <int FA, int FB> static hipError_t launch_km_fmts(const MmArgs& p, hipStream_t st) {
  switch (p.layout) {
    case 1: return launch_dma_family<FA, FB, -1, 1>(p, st);
    case 2: return launch_dma_family<FA, FB, -1, 2>(p, st);
    default: return launch_dma_family<FA, FB, -1, 3>(p, st);
  }
}

hipError_t launch_mm_km(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st) {
  if (mm_precise(p)) return launch_mm_prec_km(p, fmt_a, fmt_b, st);
  if (fmt_a == kE4M3 && fmt_b == kE4M3) return launch_km_fmts<kE4M3, kE4M3>(p, st);
  if (fmt_a == kE5M2 && fmt_b == kE4M3) return launch_km_fmts<kE5M2, kE4M3>(p, st);
  if (fmt_a == kE4M3 && fmt_b == kE5M2) return launch_km_fmts<kE4M3, kE5M2>(p, st);
  return launch_km_fmts<kE5M2, kE5M2>(p, st);
}

}  // namespace fp8mi
