// Host-side internal interface between the C ABI layer and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8mi {

// Compute-unit count of the current device (cached per device).
int device_cu_count();

// Integer tuning override from the environment: the value of `name` when it
// is a decimal integer in [lo, hi], else dflt (unset, malformed or out of
// range values are ignored).
int env_int_in(const char* name, int lo, int hi, int dflt);

// mode: 0 row, 1 transposed, 2 dual.  Arguments already validated.  With
// bias_ws (dual, bf16/fp16 input) the dual kernel also writes fp64 column sums
// per 128-row tile to bias_ws[tile row][col] (the grad_bias workspace layout).
hipError_t launch_quantize(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld_x, int fmt, int mode,
                           uint8_t* out_row, int64_t ld_row, uint8_t* out_t, int64_t ld_t, const float* scale,
                           uint32_t* ring, int H, float* scale_inv_out, float* amax_out, hipStream_t st,
                           double* bias_ws = nullptr);

// Current scaling: amax partials into `parts` (kDynWorkspaceBytes bytes, one
// fp32 word per partial), then the quantize with s = fmt_max / amax.
// Arguments validated.
constexpr int64_t kDynWorkspaceBytes = 4096;
hipError_t launch_quantize_dynamic(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                                   int mode, uint8_t* out_row, int64_t ld_row, uint8_t* out_t, int64_t ld_t,
                                   float* scale_inv_out, float* amax_out, uint32_t* parts, hipStream_t st);

hipError_t launch_amax_fold(uint32_t* ring, int H, const float* amax, int fmt, hipStream_t st);

struct MmArgs {
  const uint8_t* a = nullptr;
  const uint8_t* b = nullptr;
  int64_t lda = 0, ldb = 0, stride_a = 0, stride_b = 0;
  int64_t M = 0, N = 0, K = 0, batch = 0;
  const float* a_scale_inv = nullptr;
  const float* b_scale_inv = nullptr;
  const void* bias = nullptr;
  int bias_dtype = -1;                // -1: no bias; kF32 / kF16 / kBF16; kFp8E4M3 / kFp8E5M2 codes
  const float* bias_scale = nullptr;  // dequantisation multiplier of an fp8 bias
  void* c = nullptr;                  // bf16 (out_fmt < 0) or fp8 codes (out_fmt = kE4M3 / kE5M2)
  int64_t ldc = 0, stride_c = 0;      // elements
  int out_fmt = -1;
  // fp8 output: scale from c_scale or the ring c_ring (history c_H); optional 1/s and amax outputs
  const float* c_scale = nullptr;
  uint32_t* c_ring = nullptr;
  int c_H = 0;
  float* c_scale_inv_out = nullptr;
  float* c_amax_out = nullptr;
  int layout = 0;                     // bit 0: A is [K, M] (K-major), bit 1: B is [K, N]
  int early_loads = 0;                // set by the launch: big tiles issue a K step's loads early

  // Bytes of one batch's A (B) from row r on: the last row ends at K.
  __host__ __device__ int64_t a_extent_from(int64_t r) const { return r < M ? (M - 1 - r) * lda + K : 0; }
  __host__ __device__ int64_t b_extent_from(int64_t r) const { return r < N ? (N - 1 - r) * ldb + K : 0; }
  // K-major operands ([K, ld] arrays of K full rows): bytes from column r of
  // row 0 to the end of row K - 1 including its padding, so the extent ends
  // on a 16-byte chunk boundary (lda % 16 == 0, r % 16 == 0): the raw-buffer
  // range check zeroes a straddling 16-byte access as a whole.
  __host__ __device__ int64_t a_extent_km(int64_t r) const { return (r < M && K > 0) ? K * lda - r : 0; }
  __host__ __device__ int64_t b_extent_km(int64_t r) const { return (r < N && K > 0) ? K * ldb - r : 0; }
};

hipError_t launch_mm(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st);
// fp8-output GEMM (p.out_fmt >= 0, either layout, operand extents below 2^31 bytes).
hipError_t launch_mm_q8(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st);
// bf16-output GEMM with K-major operand(s) (p.layout != 0, extents below 2^31 bytes).
hipError_t launch_mm_km(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st);
// fp8-output GEMM with K-major operand(s), one per layout tag (1: A, 2: B,
// 3: both), called by launch_mm_q8.
hipError_t launch_mm_km_q8_l1(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st);
hipError_t launch_mm_km_q8_l2(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st);
hipError_t launch_mm_km_q8_l3(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st);
// Short K (K <= kPreciseMaxK, mm_fp8_kernel.h): the precise-accumulation
// kernels, bf16 NT / bf16 K-major / fp8 output NT / fp8 output K-major
// (operand extents below 2^31 bytes).
hipError_t launch_mm_prec_nt(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st);
hipError_t launch_mm_prec_km(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st);
hipError_t launch_mm_prec_q8(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st);
hipError_t launch_mm_prec_km_q8(const MmArgs& p, int fmt_a, int fmt_b, hipStream_t st);
// One fp32 word set to 0 on the stream (a fill kernel, capturable).
hipError_t launch_zero_word(float* p, hipStream_t st);

// Bytes of fp64 workspace the bias gradient needs (per-chunk column sums).
int64_t grad_bias_workspace_bytes(int64_t rows, int64_t cols);
hipError_t launch_grad_bias(const void* dy, int dt, int64_t rows, int64_t cols, int64_t ld, uint16_t* out,
                            void* workspace, hipStream_t st);
// Second half of the bias gradient: adds the per-chunk sums in chunk order, one bf16 rounding.
hipError_t launch_grad_bias_finalize(const double* ws, int64_t rows, int64_t cols, uint16_t* out, hipStream_t st);
hipError_t launch_ring_seed(uint32_t* ring, int H, const float* amax, int fmt, hipStream_t st);
// Measurement aid (stream.hip): read src_bytes, write dst_bytes (= src_bytes or its half).
hipError_t launch_stream(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes, hipStream_t st);

}  // namespace fp8mi
