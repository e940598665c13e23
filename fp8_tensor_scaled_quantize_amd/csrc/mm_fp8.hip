// Per-tensor-scaled fp8 GEMM on CDNA4 MFMA (gfx950), NT operands, fp32
// accumulation, fused fp32 bias, one bf16 rounding of the output, batched
// through grid.z with optional stride-0 broadcast.  The kernel template lives
// in mm_fp8_kernel.h; this unit holds the bf16-output NT instantiations, the
// plain-load fallback and the dispatch, mm_fp8_q8.hip the fp8-output ones
// (the quantizing epilogue) and mm_fp8_km.hip the K-major ones (layout tags).
//
// log:tests/extension -- the commit fusing the linear bias into the GEMM
// epilogue (added in fp32 before the single bf16 rounding, guarded N tails,
// batch broadcast from the row-major layout); the commit accepting 3-D
// operands (grid.z over batch strides, size-1 batches broadcast at stride 0);
// the commit making the GEMM output always bf16.
// log:csrc/kernels/fp8_mm.cu, commit 5244f1a8fc -- per-tensor scales applied
// inside the GEMM (dequantisation multipliers for A and B).
//
// Kernel shape on MI355X: v_mfma_f32_16x16x128_f8f6f4 (no block scales) with
// the A/B formats selected by cbsz/blgp.
// The operands are swapped at the MFMA (B rows drive the instruction's first
// operand), so each lane ends with 4 consecutive output columns of one row
// and writes 8 contiguous bytes of bf16.  LDS tiles hold 128 K-bytes per row,
// 16-byte chunks XOR-swizzled (see swz) so that the 16 rows one MFMA
// fragment reads spread over the banks.
#include "mm_fp8_kernel.h"

namespace fp8mi {

template <int BM, int BN, int FA, int FB, bool PREC>
__global__ void __launch_bounds__(kMmThreads) mm_fp8_tile(MmArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2;             // 2 x 2 waves
  constexpr int TI = WM / 16, TJ = WN / 16;           // MFMA tiles per wave
  constexpr int CA = BM * (kBK / 16) / kMmThreads;    // 16-byte chunks per thread
  constexpr int CB = BN * (kBK / 16) / kMmThreads;
  static_assert(CA >= 1 && CB >= 1, "tile too small for the thread count");
  __shared__ __align__(16) uint8_t As[BM * kBK];
  __shared__ __align__(16) uint8_t Bs[BN * kBK];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int64_t bz = blockIdx.z;
  const uint8_t* A = p.a + bz * p.stride_a;
  const uint8_t* B = p.b + bz * p.stride_b;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;

  uint4 ra[CA], rb[CB];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int id = tid + kMmThreads * i, row = id >> 3, ch = id & 7;
      const int64_t gm = m0 + row, gk = k0 + 16 * ch;
      ra[i] = (gm < p.M && gk < p.K) ? *reinterpret_cast<const uint4*>(A + gm * p.lda + gk) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int id = tid + kMmThreads * i, row = id >> 3, ch = id & 7;
      const int64_t gn = n0 + row, gk = k0 + 16 * ch;
      rb[i] = (gn < p.N && gk < p.K) ? *reinterpret_cast<const uint4*>(B + gn * p.ldb + gk) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int id = tid + kMmThreads * i, row = id >> 3, ch = id & 7;
      *reinterpret_cast<uint4*>(As + row * kBK + ((ch ^ swz(row)) << 4)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int id = tid + kMmThreads * i, row = id >> 3, ch = id & 7;
      *reinterpret_cast<uint4*>(Bs + row * kBK + ((ch ^ swz(row)) << 4)) = rb[i];
    }
  };

  v4f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t nk = (p.K + kBK - 1) / kBK;
  if (nk > 0) {
    gload(0);
    sstore();
  }
  __syncthreads();
  const int r16 = lane & 15, g = lane >> 4;
  for (int64_t kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload((kt + 1) * kBK);
    v8i af[TI], bfr[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) af[i] = lds_frag(As, wm * WM + 16 * i + r16, g);
#pragma unroll
    for (int j = 0; j < TJ; ++j) bfr[j] = lds_frag(Bs, wn * WN + 16 * j + r16, g);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = mma<FA, FB, PREC>(bfr[j], af[i], acc[i][j]);
    __syncthreads();
    if (kt + 1 < nk) {
      sstore();
      __syncthreads();
    }
  }

  // Epilogue: y = acc * fl32(sa * sb) + bias[j], one bf16 rounding.
  const float sa = p.a_scale_inv ? *p.a_scale_inv : 1.0f;
  const float sb = p.b_scale_inv ? *p.b_scale_inv : 1.0f;
  const float sab = sa * sb;
  const float bscale = p.bias_scale ? *p.bias_scale : 1.0f;
  uint16_t* C = static_cast<uint16_t*>(p.c) + bz * p.stride_c;
  const int mr = lane & 15, ng = lane >> 4;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int64_t gm = m0 + wm * WM + 16 * i + mr;
    if (gm >= p.M) continue;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t gn = n0 + wn * WN + 16 * j + 4 * ng;
      if (gn >= p.N) continue;
      float y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float bv = (p.bias && gn + r < p.N) ? load_bias(p, gn + r, bscale) : 0.0f;
        y[r] = fmaf(acc[i][j][r], sab, bv);
      }
      const uint2 w = bf16x4_rne(y[0], y[1], y[2], y[3]);
      const uint32_t h[4] = {w.x & 0xFFFFu, w.x >> 16, w.y & 0xFFFFu, w.y >> 16};
      uint16_t* dst = C + gm * p.ldc + gn;
      if (gn + 4 <= p.N && ((reinterpret_cast<uintptr_t>(dst) & 7u) == 0)) {
        *reinterpret_cast<uint2*>(dst) = w;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (gn + r < p.N) dst[r] = (uint16_t)h[r];
      }
    }
  }
}

// Large operands (byte extents beyond a 32-bit buffer offset) take the
// 128x128 plain-load kernel; everything else the LDS-DMA big-tile family.
// Short K takes the precise accumulation in either case.
template <int FA, int FB> static hipError_t launch_fmts(const MmArgs& p, hipStream_t st) {
  if (mm_fits31(p)) return mm_precise(p) ? launch_mm_prec_nt(p, FA, FB, st) : launch_dma_family<FA, FB, -1>(p, st);
  constexpr int BM = 128, BN = 128;
  const dim3 grid((unsigned)((p.N + BN - 1) / BN), (unsigned)((p.M + BM - 1) / BM), (unsigned)p.batch);
  if (mm_precise(p))
    hipLaunchKernelGGL((mm_fp8_tile<BM, BN, FA, FB, true>), grid, dim3(kMmThreads), 0, st, p);
  else
    hipLaunchKernelGGL((mm_fp8_tile<BM, BN, FA, FB, false>), grid, dim3(kMmThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_mm(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st) {
  if (p.out_fmt >= 0) return launch_mm_q8(p, fmt_a, fmt_b, st);
  if (p.layout != 0) return launch_mm_km(p, fmt_a, fmt_b, st);
  if (fmt_a == kE4M3 && fmt_b == kE4M3) return launch_fmts<kE4M3, kE4M3>(p, st);
  if (fmt_a == kE5M2 && fmt_b == kE4M3) return launch_fmts<kE5M2, kE4M3>(p, st);
  if (fmt_a == kE4M3 && fmt_b == kE5M2) return launch_fmts<kE4M3, kE5M2>(p, st);
  return launch_fmts<kE5M2, kE5M2>(p, st);
}

}  // namespace fp8mi
