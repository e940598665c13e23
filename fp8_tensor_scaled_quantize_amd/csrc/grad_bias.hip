// Bias gradient of an fp8 linear layer: db[j] = sum_i dY[i, j] over every
// leading dimension, returned in bf16 (log:tests/extension, the commits that
// reduce grad_b over the leading dims of 3-D inputs and keep gradients bf16).
//
// The sum runs in fp64 in a fixed order and is rounded once to bf16.  For
// bf16/fp16 inputs the fp64 partial sums are exact unless the values span more
// than ~(53 - 8 - log2 rows) binades, so the result is normally the exactly
// rounded column sum.
//
// Shape on MI355X: one workgroup of 16 waves per 64-column strip; lane l of a
// wave reads 16 bytes (8 columns) of row (l / 8) of an 8-row group, so every
// load instruction covers 8 full 128-byte row segments; waves take interleaved
// 8-row groups, each lane keeps 8 fp64 sums, and the strip reduces through
// shuffles and LDS.  No workspace, no atomics.
#include "fp8mi_device.h"
#include "fp8mi_internal.h"

namespace fp8mi {

constexpr int kGbThreads = 1024;
constexpr int kGbCols = 64;

// fp64 -> bf16, one round-to-nearest-even (no detour through fp32).
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double d) {
  const uint64_t u = __double_as_longlong(d);
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  const int e = (int)((u >> 52) & 0x7FF);
  if (e == 0x7FF) return (u & 0xFFFFFFFFFFFFFull) ? (sign | 0x7FC0u) : (sign | 0x7F80u);
  const double a = __longlong_as_double(u & 0x7FFFFFFFFFFFFFFFull);
  if (a == 0.0) return sign;
  // spacing of bf16 at |d|: 2^(max(floor(log2|d|), -126) - 7)
  int ex = e - 1023;  // exact for normal fp64; fp64 subnormals are below every bf16 step
  if (ex < -126) ex = -126;
  const double q = ldexp(1.0, ex - 7);
  const double r = rint(a / q) * q;  // a / q is exact (power-of-two scaling)
  if (r >= 0x1p128) return sign | 0x7F80u;
  return sign | (__float_as_uint((float)r) >> 16);  // r is a bf16 value: exact in fp32
}

template <int DT>
__global__ void __launch_bounds__(kGbThreads) grad_bias_kernel(const void* dy, int64_t rows, int64_t cols,
                                                               int64_t ld, uint16_t* out) {
  __shared__ double part[kGbThreads / 64][kGbCols];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  constexpr int NW = kGbThreads / 64;
  const int64_t c0 = (int64_t)blockIdx.x * kGbCols;
  const int lr = lane >> 3, lg = lane & 7;  // row within the 8-row group, 8-column group
  const int64_t cc = c0 + 8 * lg;
  const char* base = static_cast<const char*>(dy);
  double s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const bool vec = cc + 8 <= cols && (ld % 8) == 0 && ((reinterpret_cast<uintptr_t>(dy) & 15u) == 0);
  for (int64_t r = (int64_t)wid * 8 + lr; r < rows; r += NW * 8) {
    if (vec) {
      const uint4 v = *reinterpret_cast<const uint4*>(base + (r * ld + cc) * 2);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float lo, hi;
        widen2<DT>(w[e], lo, hi);
        s[2 * e] += (double)lo;
        s[2 * e + 1] += (double)hi;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (cc + e < cols) s[e] += (double)load1<DT>(dy, r * ld + cc + e);
    }
  }
  // reduce the 8 row-lanes (lanes with equal lg) of the wave
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    double v = s[e];
    v += __shfl_xor(v, 8, 64);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    s[e] = v;
  }
  if (lr == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) part[wid][8 * lg + e] = s[e];
  }
  __syncthreads();
  if (threadIdx.x < kGbCols) {
    const int64_t c = c0 + threadIdx.x;
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += part[w][threadIdx.x];
    if (c < cols) out[c] = (uint16_t)f64_to_bf16_rne(t);
  }
}

hipError_t launch_grad_bias(const void* dy, int dt, int64_t rows, int64_t cols, int64_t ld, uint16_t* out,
                            hipStream_t st) {
  const dim3 grid((unsigned)((cols + kGbCols - 1) / kGbCols));
  if (dt == kF16)
    hipLaunchKernelGGL((grad_bias_kernel<kF16>), grid, dim3(kGbThreads), 0, st, dy, rows, cols, ld, out);
  else
    hipLaunchKernelGGL((grad_bias_kernel<kBF16>), grid, dim3(kGbThreads), 0, st, dy, rows, cols, ld, out);
  return hipGetLastError();
}

// Ring seed: history and scratch cleared, slot 0, and the scale a fold of
// `amax` into an empty window publishes (fmt_max / amax, or 1.0).
template <int FMT> __global__ void ring_seed_kernel(uint32_t* ring, int H, const float* amax) {
  const int t = threadIdx.x;
  for (int i = t; i < H + 4 + kFoldSlots * kFoldSlotStride; i += blockDim.x)
    if (i != H) ring[i] = 0u;
  if (t == 0) {
    const float m = *amax;
    float s = 1.0f;
    if (m > 0.0f && m <= 3.40282347e38f) {
      const float q = FmtTraits<FMT>::kMax / m;
      if (q > 0.0f && q <= 3.40282347e38f) s = q;
    }
    ring[H] = __float_as_uint(s);
  }
}

hipError_t launch_ring_seed(uint32_t* ring, int H, const float* amax, int fmt, hipStream_t st) {
  if (fmt == kE4M3) hipLaunchKernelGGL(ring_seed_kernel<kE4M3>, dim3(1), dim3(256), 0, st, ring, H, amax);
  else hipLaunchKernelGGL(ring_seed_kernel<kE5M2>, dim3(1), dim3(256), 0, st, ring, H, amax);
  return hipGetLastError();
}

}  // namespace fp8mi
