// Streaming reference kernel for measurement: the HBM traffic of a quantize
// with none of its arithmetic.  It reads every byte of src once and writes
// every byte of dst once with the row quantize's access shape (16-byte loads
// per lane, 256 threads, four loads of one workgroup's 16 KiB share in flight
// per lane before any store), so its time is the practical ceiling a
// quantize of the same bytes can approach on this GPU.  dst gets bytes taken
// from the loaded data (the high byte of each 16-bit pair when dst is half of
// src, the data itself when the sizes match), so no load can be dropped.
#include "fp8mi_device.h"
#include "fp8mi_internal.h"

namespace fp8mi {

constexpr int kStreamThreads = 256;
constexpr int kStreamLoads = 4;  // 16-byte loads per lane in flight

template <bool HALF>
__global__ void __launch_bounds__(kStreamThreads) stream_kernel(const uint4* src, int64_t nchunks, void* dst) {
  const int64_t base = (int64_t)blockIdx.x * (kStreamThreads * kStreamLoads) + threadIdx.x;
  uint4 v[kStreamLoads];
#pragma unroll
  for (int i = 0; i < kStreamLoads; ++i) {
    const int64_t c = base + (int64_t)i * kStreamThreads;
    v[i] = c < nchunks ? src[c] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < kStreamLoads; ++i) {
    const int64_t c = base + (int64_t)i * kStreamThreads;
    if (c >= nchunks) continue;
    if constexpr (HALF) {
      // byte 1 of each 16-bit pair: the top byte of a bf16 / fp16 element
      const uint32_t lo = __builtin_amdgcn_perm(v[i].y, v[i].x, 0x07050301u);
      const uint32_t hi = __builtin_amdgcn_perm(v[i].w, v[i].z, 0x07050301u);
      static_cast<uint2*>(dst)[c] = make_uint2(lo, hi);
    } else {
      static_cast<uint4*>(dst)[c] = v[i];
    }
  }
}

hipError_t launch_stream(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes, hipStream_t st) {
  const int64_t nchunks = src_bytes / 16;
  if (nchunks == 0) return hipSuccess;
  const int64_t per_block = (int64_t)kStreamThreads * kStreamLoads;
  const dim3 grid((unsigned)((nchunks + per_block - 1) / per_block));
  if (dst_bytes == src_bytes)
    hipLaunchKernelGGL(stream_kernel<false>, grid, dim3(kStreamThreads), 0, st, static_cast<const uint4*>(src),
                       nchunks, dst);
  else
    hipLaunchKernelGGL(stream_kernel<true>, grid, dim3(kStreamThreads), 0, st, static_cast<const uint4*>(src),
                       nchunks, dst);
  return hipGetLastError();
}

}  // namespace fp8mi
