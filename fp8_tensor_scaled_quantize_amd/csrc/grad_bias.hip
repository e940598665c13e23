// Bias gradient of an fp8 linear layer: db[j] = sum_i dY[i, j] over every
// leading dimension, returned in bf16 (log:tests/extension, the commits that
// reduce grad_b over the leading dims of 3-D inputs and keep gradients bf16).
//
// The sum runs in fp64 in a fixed order and is rounded once to bf16.  For
// bf16/fp16 inputs the fp64 partial sums are exact unless the values span more
// than ~(53 - 8 - log2 rows) binades, so the result is normally the exactly
// rounded column sum.
//
// Shape on MI355X: two launches over a caller-provided fp64 workspace.
//  * partials: a 2-D grid of (512-column block, 128-row chunk) workgroups of
//    4 waves.  Lane l owns columns 8l .. 8l + 7 of the block, so every load
//    instruction reads one contiguous 1 KiB row segment; wave w sums rows
//    w, w + 4, ... of the chunk in order, the 4 waves combine through LDS in
//    wave order, and the chunk's column sums go to workspace[chunk][col].
//  * finalize: 8 sub-lanes per column each add a contiguous range of chunks
//    in chunk order, the 8 partials are added in sub-lane order, and the
//    total is rounded once to bf16.
// Every sum has a fixed order, so the result does not depend on scheduling,
// and the grid (cols / 512 x rows / 128 workgroups) fills the chip even for
// the few thousand columns of a linear layer.
#include "fp8mi_device.h"
#include "fp8mi_internal.h"

namespace fp8mi {

constexpr int kGbThreads = 256;
constexpr int kGbCols = 512;        // columns per workgroup (64 lanes x 8)
constexpr int kGbRowChunk = 128;    // rows per workgroup

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
__global__ void __launch_bounds__(kGbThreads) grad_bias_partials(const void* dy, int64_t rows, int64_t cols,
                                                                 int64_t ld, double* ws) {
  __shared__ double part[kGbThreads / 64][kGbCols];
  constexpr int NW = kGbThreads / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kGbCols;
  const int64_t cc = c0 + 8 * lane;
  const int64_t r0 = (int64_t)blockIdx.y * kGbRowChunk;
  const int64_t r1 = r0 + kGbRowChunk < rows ? r0 + kGbRowChunk : rows;
  const char* base = static_cast<const char*>(dy);
  double s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const bool vec = cc + 8 <= cols && (ld % 8) == 0 && ((reinterpret_cast<uintptr_t>(dy) & 15u) == 0);
  if (vec) {
    auto add_row = [&](const uint4& v) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float lo, hi;
        widen2<DT>(w[e], lo, hi);
        s[2 * e] += (double)lo;
        s[2 * e + 1] += (double)hi;
      }
    };
    // 8 rows' loads in flight before any is added (rows still added in order)
    constexpr int U = 8;
    int64_t r = r0 + wid;
    for (; r + (U - 1) * NW < r1; r += U * NW) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const uint4*>(base + ((r + u * NW) * ld + cc) * 2);
#pragma unroll
      for (int u = 0; u < U; ++u) add_row(v[u]);
    }
    for (; r < r1; r += NW) add_row(*reinterpret_cast<const uint4*>(base + (r * ld + cc) * 2));
  } else {
    for (int64_t r = r0 + wid; r < r1; r += NW) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (cc + e < cols) s[e] += (double)load1<DT>(dy, r * ld + cc + e);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[wid][8 * lane + e] = s[e];
  __syncthreads();
  for (int c = threadIdx.x; c < kGbCols; c += kGbThreads) {
    const int64_t col = c0 + c;
    if (col < cols) {
      double t = part[0][c];
#pragma unroll
      for (int w = 1; w < NW; ++w) t += part[w][c];
      ws[(int64_t)blockIdx.y * cols + col] = t;
    }
  }
}

// 32 columns per workgroup, 8 sub-lanes per column: sub-lane q adds chunks
// [q * per, (q + 1) * per) in order, then the 8 partial sums are added in
// sub-lane order (threads 32q .. 32q + 31 read 32 consecutive columns).
constexpr int kGbFinCols = 32, kGbFinSplit = 8;
__global__ void __launch_bounds__(kGbFinCols * kGbFinSplit) grad_bias_finalize(const double* ws, int64_t nchunk,
                                                                               int64_t cols, uint16_t* out) {
  __shared__ double red[kGbFinSplit][kGbFinCols];
  const int c = threadIdx.x % kGbFinCols, q = threadIdx.x / kGbFinCols;
  const int64_t col = (int64_t)blockIdx.x * kGbFinCols + c;
  const int64_t per = (nchunk + kGbFinSplit - 1) / kGbFinSplit;
  const int64_t k0 = q * per, k1 = k0 + per < nchunk ? k0 + per : nchunk;
  double t = 0.0;
  if (col < cols) {
#pragma unroll 8
    for (int64_t k = k0; k < k1; ++k) t += ws[k * cols + col];
  }
  red[q][c] = t;
  __syncthreads();
  if (q == 0 && col < cols) {
    double v = red[0][c];
#pragma unroll
    for (int j = 1; j < kGbFinSplit; ++j) v += red[j][c];
    out[col] = (uint16_t)f64_to_bf16_rne(v);
  }
}

int64_t grad_bias_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  return ((rows + kGbRowChunk - 1) / kGbRowChunk) * cols * (int64_t)sizeof(double);
}

hipError_t launch_grad_bias(const void* dy, int dt, int64_t rows, int64_t cols, int64_t ld, uint16_t* out,
                            void* workspace, hipStream_t st) {
  const int64_t nchunk = rows > 0 ? (rows + kGbRowChunk - 1) / kGbRowChunk : 0;
  double* ws = static_cast<double*>(workspace);
  if (nchunk > 0) {
    const dim3 grid((unsigned)((cols + kGbCols - 1) / kGbCols), (unsigned)nchunk);
    if (dt == kF16)
      hipLaunchKernelGGL((grad_bias_partials<kF16>), grid, dim3(kGbThreads), 0, st, dy, rows, cols, ld, ws);
    else
      hipLaunchKernelGGL((grad_bias_partials<kBF16>), grid, dim3(kGbThreads), 0, st, dy, rows, cols, ld, ws);
  }
  return launch_grad_bias_finalize(ws, rows, cols, out, st);
}

hipError_t launch_grad_bias_finalize(const double* ws, int64_t rows, int64_t cols, uint16_t* out, hipStream_t st) {
  const int64_t nchunk = rows > 0 ? (rows + kGbRowChunk - 1) / kGbRowChunk : 0;
  hipLaunchKernelGGL(grad_bias_finalize, dim3((unsigned)((cols + kGbFinCols - 1) / kGbFinCols)),
                     dim3(kGbFinCols * kGbFinSplit), 0, st, ws, nchunk, cols, out);
  return hipGetLastError();
}

// Ring seed: history and scratch cleared, slot 0, and the scale a fold of
// `amax` into an empty window publishes (fmt_max / amax, or 1.0).
template <int FMT> __global__ void ring_seed_kernel(uint32_t* ring, int H, const float* amax) {
  const int t = threadIdx.x;
  for (int i = t; i < H + 4 + kFoldSlots * kFoldSlotStride; i += blockDim.x)
    if (i != H) ring[i] = 0u;
  if (t == 0) {
    ring[H] = __float_as_uint(scale_from_max<FMT>(*amax));
  }
}

hipError_t launch_ring_seed(uint32_t* ring, int H, const float* amax, int fmt, hipStream_t st) {
  if (fmt == kE4M3) hipLaunchKernelGGL(ring_seed_kernel<kE4M3>, dim3(1), dim3(256), 0, st, ring, H, amax);
  else hipLaunchKernelGGL(ring_seed_kernel<kE5M2>, dim3(1), dim3(256), 0, st, ring, H, amax);
  return hipGetLastError();
}

}  // namespace fp8mi
