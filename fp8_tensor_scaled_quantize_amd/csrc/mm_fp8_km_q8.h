// FP8-out GEMM with layout tags: the quantizing epilogue of mm_fp8_q8.hip on
// K-major operand(s) (the layout tags of mm_fp8_km.hip).  Same tile family
// and dispatch as the NT FP8-out GEMM; every output's K sum runs in the same
// MFMA order, so codes, amax and the ring fold equal the NT form's bit for
// bit.  One translation unit per layout tag (mm_fp8_km_q8_{a,b,ab}.hip), so
// the build compiles the three in parallel.
#pragma once
#include "mm_fp8_kernel.h"

namespace fp8mi {

template <int LAY> hipError_t launch_mm_km_q8_layout(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st) {
  const bool e4 = p.out_fmt == kE4M3;
  if (fmt_a == kE4M3 && fmt_b == kE4M3)
    return e4 ? launch_dma_family<kE4M3, kE4M3, kE4M3, LAY>(p, st) : launch_dma_family<kE4M3, kE4M3, kE5M2, LAY>(p, st);
  if (fmt_a == kE5M2 && fmt_b == kE4M3)
    return e4 ? launch_dma_family<kE5M2, kE4M3, kE4M3, LAY>(p, st) : launch_dma_family<kE5M2, kE4M3, kE5M2, LAY>(p, st);
  if (fmt_a == kE4M3 && fmt_b == kE5M2)
    return e4 ? launch_dma_family<kE4M3, kE5M2, kE4M3, LAY>(p, st) : launch_dma_family<kE4M3, kE5M2, kE5M2, LAY>(p, st);
  return e4 ? launch_dma_family<kE5M2, kE5M2, kE4M3, LAY>(p, st) : launch_dma_family<kE5M2, kE5M2, kE5M2, LAY>(p, st);
}

}  // namespace fp8mi
