// FP8-in / FP8-out GEMM: the mm_fp8_dma kernels instantiated with the
// quantizing epilogue (log:tests/extension -- the commit adding the
// FP8-in/FP8-out GEMM op; the commit giving the bias a bias_scale slot, an
// fp8-stored bias dequantized after the operand scaling and before the output
// quantization).  y = acc * fl32(sa * sb) + bias in fp32, codes
// enc(fl32(y * s_c)) with the quantize kernels' encoder, amax over the valid
// outputs published with the same slot protocol as the quantize kernels (the
// last workgroup folds into the output's ring), or atomically maxed into a
// caller word when the scale is explicit.
#include "mm_fp8_kernel.h"

namespace fp8mi {

// An empty output still completes the call's scale bookkeeping: with a ring
// it folds amax 0 (as an empty quantize does); otherwise it writes 1 / s and
// amax 0.
template <int FMT>
__global__ void mm_empty_out_kernel(uint32_t* ring, int H, const float* scale, float* scale_inv_out,
                                    float* amax_out) {
  if (threadIdx.x >= 64) return;
  if (ring) {
    ring_fold_wave<FMT>(ring, H, 0.0f, scale_inv_out, __uint_as_float(ring[H]), amax_out);
  } else if (threadIdx.x == 0) {
    if (scale_inv_out) *scale_inv_out = 1.0f / *scale;
    if (amax_out) *amax_out = 0.0f;
  }
}

template <int FA, int FB> static hipError_t launch_out(const MmArgs& p, hipStream_t st) {
  return p.out_fmt == kE4M3 ? launch_dma_family<FA, FB, kE4M3>(p, st) : launch_dma_family<FA, FB, kE5M2>(p, st);
}

hipError_t launch_mm_q8(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st) {
  if (p.M == 0 || p.N == 0 || p.batch == 0) {
    if (p.out_fmt == kE4M3)
      hipLaunchKernelGGL(mm_empty_out_kernel<kE4M3>, dim3(1), dim3(64), 0, st, p.c_ring, p.c_H, p.c_scale,
                         p.c_scale_inv_out, p.c_amax_out);
    else
      hipLaunchKernelGGL(mm_empty_out_kernel<kE5M2>, dim3(1), dim3(64), 0, st, p.c_ring, p.c_H, p.c_scale,
                         p.c_scale_inv_out, p.c_amax_out);
    return hipGetLastError();
  }
  if (!p.c_ring && p.c_amax_out) {
    const hipError_t e = launch_zero_word(p.c_amax_out, st);
    if (e != hipSuccess) return e;
  }
  if (p.layout != 0) {
    if (mm_precise(p)) return launch_mm_prec_km_q8(p, fmt_a, fmt_b, st);
    if (p.layout == 1) return launch_mm_km_q8_l1(p, fmt_a, fmt_b, st);
    if (p.layout == 2) return launch_mm_km_q8_l2(p, fmt_a, fmt_b, st);
    return launch_mm_km_q8_l3(p, fmt_a, fmt_b, st);
  }
  if (mm_precise(p)) return launch_mm_prec_q8(p, fmt_a, fmt_b, st);
  if (fmt_a == kE4M3 && fmt_b == kE4M3) return launch_out<kE4M3, kE4M3>(p, st);
  if (fmt_a == kE5M2 && fmt_b == kE4M3) return launch_out<kE5M2, kE4M3>(p, st);
  if (fmt_a == kE4M3 && fmt_b == kE5M2) return launch_out<kE4M3, kE5M2>(p, st);
  return launch_out<kE5M2, kE5M2>(p, st);
}

}  // namespace fp8mi
