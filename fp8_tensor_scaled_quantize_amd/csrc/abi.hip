// C ABI of libfp8mi: argument validation, status reporting and dispatch to
// the kernel launchers.  Every check runs before any HIP call, so a rejected
// call has no side effects.
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/fp8mi.h"
#include "fp8mi_internal.h"

namespace fp8mi {

static thread_local char g_err[512] = "";

static fp8mi_status fail(fp8mi_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

static fp8mi_status from_hip(hipError_t e, const char* where) {
  if (e == hipSuccess) return FP8MI_OK;
  return fail(FP8MI_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

int env_int_in(const char* name, int lo, int hi, int dflt) {
  const char* e = getenv(name);
  if (!e || !*e) return dflt;
  char* end = nullptr;
  const long v = strtol(e, &end, 10);
  return (*end == '\0' && v >= lo && v <= hi) ? (int)v : dflt;
}

static_assert(kDynWorkspaceBytes == FP8MI_DYNAMIC_WORKSPACE_BYTES, "dynamic workspace size");

static bool valid_fmt(int f) { return f == FP8MI_E4M3 || f == FP8MI_E5M2; }
static bool valid_dtype(int d) { return d == FP8MI_F32 || d == FP8MI_F16 || d == FP8MI_BF16; }
static int dtype_bytes(int d) { return d == FP8MI_F32 ? 4 : 2; }

// rows x ld elements of elem bytes stay within 2^62 bytes: no allocation is
// that large, and the bound keeps every 64-bit index product in the kernels
// (and the checks below) from overflowing.
static bool span_ok(int64_t rows, int64_t ld, int64_t elem) {
  if (rows <= 0 || ld <= 0) return true;
  return ld <= (INT64_C(1) << 62) / elem / rows;
}

static fp8mi_status check_scale_ring(const float* scale, uint32_t* ring, int32_t H) {
  if ((scale == nullptr) == (ring == nullptr))
    return fail(FP8MI_ERR_ARG, "give exactly one of scale and ring (scale=%p ring=%p)", (const void*)scale,
                (void*)ring);
  if (ring) {
    if (H < 1 || H > FP8MI_MAX_HIST) return fail(FP8MI_ERR_SHAPE, "hist_len %d outside [1, %d]", H, FP8MI_MAX_HIST);
    if (reinterpret_cast<uintptr_t>(ring) & 3u) return fail(FP8MI_ERR_ARG, "ring must be 4-byte aligned");
  }
  return FP8MI_OK;
}

static fp8mi_status check_input(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld_x) {
  if (!valid_dtype(dt)) return fail(FP8MI_ERR_ENUM, "x_dtype %d is not FP8MI_F32/F16/BF16", dt);
  if (rows < 0 || cols < 0) return fail(FP8MI_ERR_SHAPE, "negative shape rows=%lld cols=%lld", (long long)rows,
                                        (long long)cols);
  if (rows > 0 && ld_x < cols) return fail(FP8MI_ERR_SHAPE, "ld_x %lld < cols %lld", (long long)ld_x, (long long)cols);
  if (!span_ok(rows, ld_x, dtype_bytes(dt)))
    return fail(FP8MI_ERR_SHAPE, "rows %lld x ld_x %lld beyond 2^62 bytes", (long long)rows, (long long)ld_x);
  if (rows > 0 && cols > 0 && x == nullptr) return fail(FP8MI_ERR_NULL, "x is NULL");
  if (reinterpret_cast<uintptr_t>(x) % dtype_bytes(dt)) return fail(FP8MI_ERR_ARG, "x not aligned to its element size");
  return FP8MI_OK;
}

static fp8mi_status check_outputs(int mode, int64_t rows, int64_t cols, const uint8_t* out_row, int64_t ld_row,
                                  const uint8_t* out_t, int64_t ld_t, const float* scale_inv_out,
                                  const float* amax_out) {
  const bool any = rows > 0 && cols > 0;
  if (mode != 1) {
    if (any && !out_row) return fail(FP8MI_ERR_NULL, "row-layout output is NULL");
    if (rows > 0 && ld_row < cols) return fail(FP8MI_ERR_SHAPE, "row-layout ld %lld < cols %lld", (long long)ld_row,
                                               (long long)cols);
  }
  if (mode != 0) {
    if (any && !out_t) return fail(FP8MI_ERR_NULL, "transposed output is NULL");
    if (cols > 0 && ld_t < rows) return fail(FP8MI_ERR_SHAPE, "transposed ld %lld < rows %lld", (long long)ld_t,
                                             (long long)rows);
  }
  if ((mode != 1 && !span_ok(rows, ld_row, 1)) || (mode != 0 && !span_ok(cols, ld_t, 1)))
    return fail(FP8MI_ERR_SHAPE, "output extent beyond 2^62 bytes");
  if (reinterpret_cast<uintptr_t>(scale_inv_out) & 3u || reinterpret_cast<uintptr_t>(amax_out) & 3u)
    return fail(FP8MI_ERR_ARG, "fp32 scalars must be 4-byte aligned");
  return FP8MI_OK;
}

static fp8mi_status check_quantize(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                                   int mode, const uint8_t* out_row, int64_t ld_row, const uint8_t* out_t,
                                   int64_t ld_t, const float* scale, uint32_t* ring, int32_t H,
                                   const float* scale_inv_out, const float* amax_out) {
  fp8mi_status s = check_input(x, dt, rows, cols, ld_x);
  if (s != FP8MI_OK) return s;
  if (!valid_fmt(fmt)) return fail(FP8MI_ERR_ENUM, "fmt %d is not FP8MI_E4M3/FP8MI_E5M2", fmt);
  s = check_scale_ring(scale, ring, H);
  if (s != FP8MI_OK) return s;
  s = check_outputs(mode, rows, cols, out_row, ld_row, out_t, ld_t, scale_inv_out, amax_out);
  if (s != FP8MI_OK) return s;
  if (reinterpret_cast<uintptr_t>(scale) & 3u) return fail(FP8MI_ERR_ARG, "fp32 scalars must be 4-byte aligned");
  return FP8MI_OK;
}

static fp8mi_status quantize_common(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                                    int mode, uint8_t* out_row, int64_t ld_row, uint8_t* out_t, int64_t ld_t,
                                    const float* scale, uint32_t* ring, int32_t H, float* scale_inv_out,
                                    float* amax_out, void* stream, double* bias_ws = nullptr) {
  fp8mi_status s = check_quantize(x, dt, rows, cols, ld_x, fmt, mode, out_row, ld_row, out_t, ld_t, scale, ring, H,
                                  scale_inv_out, amax_out);
  if (s != FP8MI_OK) return s;
  hipError_t e = launch_quantize(x, dt, rows, cols, ld_x, fmt, mode, out_row, ld_row, out_t, ld_t, scale, ring, H,
                                 scale_inv_out, amax_out, static_cast<hipStream_t>(stream), bias_ws);
  return from_hip(e, "quantize launch");
}

// Bias-gradient arguments shared by fp8_bias_grad and the fused dual
// quantizes, apart from the workspace.
static fp8mi_status check_bias_grad_args(int dt, int64_t rows, int64_t cols, const void* out) {
  if (dt == FP8MI_F32) return fail(FP8MI_ERR_UNSUPPORTED, "the bias gradient takes bf16 or fp16 gradients");
  if (cols > 0 && !out) return fail(FP8MI_ERR_NULL, "bias gradient output is NULL");
  if (reinterpret_cast<uintptr_t>(out) & 1u) return fail(FP8MI_ERR_ARG, "bias gradient output must be 2-byte aligned");
  if ((cols + 511) / 512 > 0x7FFFFFFF || (rows + 127) / 128 > 65535)
    return fail(FP8MI_ERR_UNSUPPORTED, "rows=%lld cols=%lld beyond the launch grid", (long long)rows,
                (long long)cols);
  return FP8MI_OK;
}

static fp8mi_status check_bias_grad(int dt, int64_t rows, int64_t cols, const void* out, const void* workspace,
                                    size_t workspace_bytes) {
  fp8mi_status s = check_bias_grad_args(dt, rows, cols, out);
  if (s != FP8MI_OK) return s;
  const size_t need = (size_t)grad_bias_workspace_bytes(rows, cols);
  if (need > 0 && !workspace) return fail(FP8MI_ERR_NULL, "workspace is NULL (%zu bytes needed)", need);
  if (workspace_bytes < need)
    return fail(FP8MI_ERR_ARG, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 7u) return fail(FP8MI_ERR_ARG, "workspace must be 8-byte aligned");
  return FP8MI_OK;
}

// ---------------------------------------------------------------------------
// Library-owned scratch of fp8_quantize_dual_bias_grad_noalloc: the per-tile
// fp64 column sums that fp8_quantize_dual_bias_grad keeps in the caller's
// workspace.  Every device the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: its device address comes from hipGetSymbolAddress, once
// per device with that device current, and only that address is used.
// ---------------------------------------------------------------------------
static __device__ __align__(256) double scratch[FP8MI_NOALLOC_SCRATCH_BYTES / sizeof(double)];

static fp8mi_status scratch_of_current_device(double** out) {
  static std::mutex mu;
  static std::vector<double*> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return from_hip(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(FP8MI_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    addr[dev] = static_cast<double*>(p);
  }
  *out = addr[dev];
  return FP8MI_OK;
}

}  // namespace fp8mi

using namespace fp8mi;

extern "C" {

fp8mi_status fp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                          int transposed, uint8_t* out, int64_t ld_out, const float* scale, uint32_t* ring,
                          int32_t hist_len, float* scale_inv_out, float* amax_out, void* stream) {
  if (transposed != 0 && transposed != 1) return fail(FP8MI_ERR_ENUM, "transposed must be 0 or 1, got %d", transposed);
  if (transposed)
    return quantize_common(x, x_dtype, rows, cols, ld_x, fmt, 1, nullptr, 0, out, ld_out, scale, ring, hist_len,
                           scale_inv_out, amax_out, stream);
  return quantize_common(x, x_dtype, rows, cols, ld_x, fmt, 0, out, ld_out, nullptr, 0, scale, ring, hist_len,
                         scale_inv_out, amax_out, stream);
}

fp8mi_status fp8_quantize_dynamic(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                                  int layout, uint8_t* out_row, int64_t ld_row, uint8_t* out_t, int64_t ld_t,
                                  float* scale_inv_out, float* amax_out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (layout < 0 || layout > 2) return fail(FP8MI_ERR_ENUM, "layout must be 0, 1 or 2, got %d", layout);
  fp8mi_status s = check_input(x, x_dtype, rows, cols, ld_x);
  if (s != FP8MI_OK) return s;
  if (!valid_fmt(fmt)) return fail(FP8MI_ERR_ENUM, "fmt %d is not FP8MI_E4M3/FP8MI_E5M2", fmt);
  s = check_outputs(layout, rows, cols, out_row, ld_row, out_t, ld_t, scale_inv_out, amax_out);
  if (s != FP8MI_OK) return s;
  const size_t need = (size_t)kDynWorkspaceBytes;
  if (!workspace) return fail(FP8MI_ERR_NULL, "workspace is NULL (%zu bytes needed)", need);
  if (workspace_bytes < need) return fail(FP8MI_ERR_ARG, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 3u) return fail(FP8MI_ERR_ARG, "workspace must be 4-byte aligned");
  return from_hip(launch_quantize_dynamic(x, x_dtype, rows, cols, ld_x, fmt, layout, out_row, ld_row, out_t, ld_t,
                                          scale_inv_out, amax_out, static_cast<uint32_t*>(workspace),
                                          static_cast<hipStream_t>(stream)),
                  "dynamic quantize launch");
}

fp8mi_status fp8_quantize_dual(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                               uint8_t* out_row, int64_t ld_row, uint8_t* out_t, int64_t ld_t, const float* scale,
                               uint32_t* ring, int32_t hist_len, float* scale_inv_out, float* amax_out,
                               void* stream) {
  return quantize_common(x, x_dtype, rows, cols, ld_x, fmt, 2, out_row, ld_row, out_t, ld_t, scale, ring, hist_len,
                         scale_inv_out, amax_out, stream);
}

fp8mi_status fp8_quantize_dual_bias_grad(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                         int fmt, uint8_t* out_row, int64_t ld_row, uint8_t* out_t, int64_t ld_t,
                                         const float* scale, uint32_t* ring, int32_t hist_len, float* scale_inv_out,
                                         float* amax_out, void* bias_grad_out, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  if (!valid_dtype(x_dtype)) return fail(FP8MI_ERR_ENUM, "x_dtype %d is not F32/F16/BF16", x_dtype);
  fp8mi_status s = check_bias_grad(x_dtype, rows, cols, bias_grad_out, workspace, workspace_bytes);
  if (s != FP8MI_OK) return s;
  s = quantize_common(x, x_dtype, rows, cols, ld_x, fmt, 2, out_row, ld_row, out_t, ld_t, scale, ring, hist_len,
                      scale_inv_out, amax_out, stream, static_cast<double*>(workspace));
  if (s != FP8MI_OK || cols == 0) return s;
  return from_hip(launch_grad_bias_finalize(static_cast<const double*>(workspace), rows, cols,
                                            static_cast<uint16_t*>(bias_grad_out), static_cast<hipStream_t>(stream)),
                  "bias grad finalize launch");
}

fp8mi_status fp8_quantize_dual_bias_grad_noalloc(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                                 int64_t ld_x, int fmt, uint8_t* out_row, int64_t ld_row,
                                                 uint8_t* out_t, int64_t ld_t, const float* scale, uint32_t* ring,
                                                 int32_t hist_len, float* scale_inv_out, float* amax_out,
                                                 void* bias_grad_out, void* stream) {
  if (!valid_dtype(x_dtype)) return fail(FP8MI_ERR_ENUM, "x_dtype %d is not F32/F16/BF16", x_dtype);
  fp8mi_status s = check_bias_grad_args(x_dtype, rows, cols, bias_grad_out);
  if (s != FP8MI_OK) return s;
  s = check_quantize(x, x_dtype, rows, cols, ld_x, fmt, 2, out_row, ld_row, out_t, ld_t, scale, ring, hist_len,
                     scale_inv_out, amax_out);
  if (s != FP8MI_OK) return s;
  const size_t need = (size_t)grad_bias_workspace_bytes(rows, cols);
  if (need > (size_t)FP8MI_NOALLOC_SCRATCH_BYTES)
    return fail(FP8MI_ERR_UNSUPPORTED,
                "rows=%lld cols=%lld need %zu bytes of bias-gradient scratch, above the library's %zu; "
                "use fp8_quantize_dual_bias_grad with a caller workspace",
                (long long)rows, (long long)cols, need, (size_t)FP8MI_NOALLOC_SCRATCH_BYTES);
  double* ws = nullptr;
  if (need > 0) {
    s = scratch_of_current_device(&ws);
    if (s != FP8MI_OK) return s;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  s = from_hip(launch_quantize(x, x_dtype, rows, cols, ld_x, fmt, 2, out_row, ld_row, out_t, ld_t, scale, ring,
                               hist_len, scale_inv_out, amax_out, st, ws),
               "quantize launch");
  if (s != FP8MI_OK || cols == 0) return s;
  return from_hip(launch_grad_bias_finalize(ws, rows, cols, static_cast<uint16_t*>(bias_grad_out), st),
                  "bias grad finalize launch");
}

fp8mi_status fp8_amax_fold(uint32_t* ring, int32_t hist_len, const float* amax, int fmt, void* stream) {
  if (!ring) return fail(FP8MI_ERR_NULL, "ring is NULL");
  if (!amax) return fail(FP8MI_ERR_NULL, "amax is NULL");
  if (!valid_fmt(fmt)) return fail(FP8MI_ERR_ENUM, "fmt %d is not FP8MI_E4M3/FP8MI_E5M2", fmt);
  fp8mi_status s = check_scale_ring(nullptr, ring, hist_len);
  if (s != FP8MI_OK) return s;
  return from_hip(launch_amax_fold(ring, hist_len, amax, fmt, static_cast<hipStream_t>(stream)), "fold launch");
}

fp8mi_status fp8_mm_ex(const uint8_t* a, int fmt_a, int64_t lda, int64_t stride_a, const uint8_t* b, int fmt_b,
                       int64_t ldb, int64_t stride_b, int64_t M, int64_t N, int64_t K, int64_t batch, int layout,
                       const float* a_scale_inv, const float* b_scale_inv, const void* bias, int bias_dtype,
                       const float* bias_scale, void* c, int c_dtype, int64_t ldc, int64_t stride_c,
                       const float* c_scale, uint32_t* c_ring, int32_t c_hist_len, float* c_scale_inv_out,
                       float* c_amax_out, void* stream) {
  if (!valid_fmt(fmt_a) || !valid_fmt(fmt_b))
    return fail(FP8MI_ERR_ENUM, "fmt_a %d / fmt_b %d must be FP8MI_E4M3/FP8MI_E5M2", fmt_a, fmt_b);
  if (layout < 0 || layout > 3) return fail(FP8MI_ERR_ENUM, "layout %d is not a combination of FP8MI_A_KM / FP8MI_B_KM", layout);
  const bool fp8_bias = bias_dtype == FP8MI_FP8_E4M3 || bias_dtype == FP8MI_FP8_E5M2;
  if (bias && !valid_dtype(bias_dtype) && !fp8_bias)
    return fail(FP8MI_ERR_ENUM, "bias_dtype %d is not F32/F16/BF16/FP8_E4M3/FP8_E5M2", bias_dtype);
  if (bias && fp8_bias && !bias_scale) return fail(FP8MI_ERR_NULL, "an fp8 bias needs bias_scale");
  if (bias_scale && !(bias && fp8_bias))
    return fail(FP8MI_ERR_ARG, "bias_scale is only for an fp8-stored bias (null scale = raw bias)");
  const bool fp8_out = c_dtype == FP8MI_FP8_E4M3 || c_dtype == FP8MI_FP8_E5M2;
  if (c_dtype != FP8MI_BF16 && !fp8_out) return fail(FP8MI_ERR_ENUM, "c_dtype %d is not BF16/FP8_E4M3/FP8_E5M2", c_dtype);
  if (fp8_out) {
    fp8mi_status s = check_scale_ring(c_scale, c_ring, c_hist_len);
    if (s != FP8MI_OK) return s;
  } else if (c_scale || c_ring || c_scale_inv_out || c_amax_out) {
    return fail(FP8MI_ERR_ARG, "output scale, ring, scale_inv and amax are for an fp8 output only");
  }
  if (M < 0 || N < 0 || K < 0 || batch < 0)
    return fail(FP8MI_ERR_SHAPE, "negative size M=%lld N=%lld K=%lld batch=%lld", (long long)M, (long long)N,
                (long long)K, (long long)batch);
  if ((reinterpret_cast<uintptr_t>(c_scale) | reinterpret_cast<uintptr_t>(c_scale_inv_out) |
       reinterpret_cast<uintptr_t>(c_amax_out) | reinterpret_cast<uintptr_t>(bias_scale)) & 3u)
    return fail(FP8MI_ERR_ARG, "fp32 scalars must be 4-byte aligned");
  MmArgs p;
  p.M = M; p.N = N; p.K = K; p.batch = batch;
  p.out_fmt = fp8_out ? (c_dtype == FP8MI_FP8_E4M3 ? (int)FP8MI_E4M3 : (int)FP8MI_E5M2) : -1;
  p.c_scale = c_scale; p.c_ring = c_ring; p.c_H = c_hist_len;
  p.c_scale_inv_out = c_scale_inv_out; p.c_amax_out = c_amax_out;
  if (M == 0 || N == 0 || batch == 0) {
    // nothing to compute; an fp8 output still completes its scale bookkeeping
    if (!fp8_out) return FP8MI_OK;
    return from_hip(launch_mm(p, fmt_a, fmt_b, static_cast<hipStream_t>(stream)), "mm launch");
  }
  if (!c) return fail(FP8MI_ERR_NULL, "c is NULL");
  if (K > 0 && (!a || !b)) return fail(FP8MI_ERR_NULL, "a or b is NULL");
  if (ldc < N) return fail(FP8MI_ERR_SHAPE, "ldc %lld < N %lld", (long long)ldc, (long long)N);
  const int64_t row_a = (layout & 1) ? M : K, row_b = (layout & 2) ? N : K;  // bytes per stored row
  if (K > 0 && (lda < row_a || ldb < row_b))
    return fail(FP8MI_ERR_SHAPE, "lda %lld / ldb %lld shorter than a stored row (%lld / %lld)", (long long)lda,
                (long long)ldb, (long long)row_a, (long long)row_b);
  if (stride_a < 0 || stride_b < 0 || stride_c < 0) return fail(FP8MI_ERR_STRIDE, "negative batch stride");
  const int64_t elem_c = fp8_out ? 1 : 2;
  const bool reads = K > 0;  // A and B are not read when K = 0
  if ((reads && (!span_ok((layout & 1) ? K : M, lda, 1) || !span_ok((layout & 2) ? K : N, ldb, 1) ||
                 !span_ok(batch, stride_a, 1) || !span_ok(batch, stride_b, 1))) ||
      !span_ok(M, ldc, elem_c) || !span_ok(batch, stride_c, elem_c))
    return fail(FP8MI_ERR_SHAPE, "an operand or output extent is beyond 2^62 bytes");
  if (batch > 1 && stride_c < M * ldc)
    return fail(FP8MI_ERR_STRIDE, "stride_c %lld < M*ldc %lld: batches would overlap", (long long)stride_c,
                (long long)(M * ldc));
  if (!fp8_out && (reinterpret_cast<uintptr_t>(c) & 1u)) return fail(FP8MI_ERR_ARG, "c must be 2-byte aligned");
  if (bias && !fp8_bias && (reinterpret_cast<uintptr_t>(bias) % dtype_bytes(bias_dtype)))
    return fail(FP8MI_ERR_ARG, "bias not aligned to its element size");
  if (K > 0) {
    if ((K % 16) || (lda % 16) || (ldb % 16))
      return fail(FP8MI_ERR_UNSUPPORTED, "K, lda and ldb must be multiples of 16 (K=%lld lda=%lld ldb=%lld)",
                  (long long)K, (long long)lda, (long long)ldb);
    if ((reinterpret_cast<uintptr_t>(a) & 15u) || (reinterpret_cast<uintptr_t>(b) & 15u))
      return fail(FP8MI_ERR_UNSUPPORTED, "a and b must be 16-byte aligned");
    if ((stride_a % 16) || (stride_b % 16))
      return fail(FP8MI_ERR_UNSUPPORTED, "batch strides of a and b must be multiples of 16");
  }
  // the smallest tile is 64 x 64: its count bounds every kernel's grid; below
  // 2^29 per batch, the kernels' tile arithmetic fits 32 bits (no allocation
  // of one GPU comes near: 2^29 such tiles are 4 TB of bf16 output)
  if ((M + 63) / 64 > 65535 || batch > 65535 || (N + 63) / 64 > 0x1FFFFFFF / ((M + 63) / 64))
    return fail(FP8MI_ERR_UNSUPPORTED, "M=%lld N=%lld batch=%lld beyond the launch grid", (long long)M, (long long)N,
                (long long)batch);
  p.a = a; p.b = b; p.lda = lda; p.ldb = ldb; p.stride_a = stride_a; p.stride_b = stride_b;
  p.a_scale_inv = a_scale_inv; p.b_scale_inv = b_scale_inv;
  p.bias = bias; p.bias_dtype = bias ? bias_dtype : -1; p.bias_scale = bias_scale;
  p.c = c; p.ldc = ldc; p.stride_c = stride_c;
  p.layout = layout;
  const int64_t ext_a = (layout & 1) ? p.a_extent_km(0) : p.a_extent_from(0);
  const int64_t ext_b = (layout & 2) ? p.b_extent_km(0) : p.b_extent_from(0);
  if ((fp8_out || layout != 0) && !(ext_a < (1ll << 31) && ext_b < (1ll << 31) && K < (1ll << 30)))
    return fail(FP8MI_ERR_UNSUPPORTED, "an fp8 output or a K-major operand needs operand extents below 2^31 bytes");
  return from_hip(launch_mm(p, fmt_a, fmt_b, static_cast<hipStream_t>(stream)), "mm launch");
}

fp8mi_status fp8_mm(const uint8_t* a, int fmt_a, int64_t lda, int64_t stride_a, const uint8_t* b, int fmt_b,
                    int64_t ldb, int64_t stride_b, int64_t M, int64_t N, int64_t K, int64_t batch,
                    const float* a_scale_inv, const float* b_scale_inv, const void* bias, int bias_dtype, void* c,
                    int64_t ldc, int64_t stride_c, void* stream) {
  if (bias && !valid_dtype(bias_dtype)) return fail(FP8MI_ERR_ENUM, "bias_dtype %d is not F32/F16/BF16", bias_dtype);
  return fp8_mm_ex(a, fmt_a, lda, stride_a, b, fmt_b, ldb, stride_b, M, N, K, batch, 0, a_scale_inv, b_scale_inv, bias,
                   bias_dtype, nullptr, c, FP8MI_BF16, ldc, stride_c, nullptr, nullptr, 0, nullptr, nullptr, stream);
}

size_t fp8_bias_grad_workspace_bytes(int64_t rows, int64_t cols) {
  return (size_t)fp8mi::grad_bias_workspace_bytes(rows, cols);
}

fp8mi_status fp8_bias_grad(const void* dy, int dy_dtype, int64_t rows, int64_t cols, int64_t ld, void* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dy_dtype)) return fail(FP8MI_ERR_ENUM, "dy_dtype %d is not F32/F16/BF16", dy_dtype);
  if (dy_dtype == FP8MI_F32) return fail(FP8MI_ERR_UNSUPPORTED, "fp8_bias_grad takes bf16 or fp16 gradients");
  if (rows < 0 || cols < 0) return fail(FP8MI_ERR_SHAPE, "negative shape rows=%lld cols=%lld", (long long)rows,
                                        (long long)cols);
  if (cols == 0) return FP8MI_OK;
  if (!out) return fail(FP8MI_ERR_NULL, "out is NULL");
  if (rows > 0 && !dy) return fail(FP8MI_ERR_NULL, "dy is NULL");
  if (rows > 0 && ld < cols) return fail(FP8MI_ERR_SHAPE, "ld %lld < cols %lld", (long long)ld, (long long)cols);
  if (!span_ok(rows, ld, 2)) return fail(FP8MI_ERR_SHAPE, "rows %lld x ld %lld beyond 2^62 bytes", (long long)rows,
                                         (long long)ld);
  if (reinterpret_cast<uintptr_t>(dy) & 1u) return fail(FP8MI_ERR_ARG, "dy must be 2-byte aligned");
  fp8mi_status s = check_bias_grad(dy_dtype, rows, cols, out, workspace, workspace_bytes);
  if (s != FP8MI_OK) return s;
  return from_hip(launch_grad_bias(dy, dy_dtype, rows, cols, ld, static_cast<uint16_t*>(out), workspace,
                                   static_cast<hipStream_t>(stream)),
                  "bias grad launch");
}

fp8mi_status fp8_ring_seed(uint32_t* ring, int32_t hist_len, const float* amax, int fmt, void* stream) {
  if (!ring) return fail(FP8MI_ERR_NULL, "ring is NULL");
  if (!amax) return fail(FP8MI_ERR_NULL, "amax is NULL");
  if (!valid_fmt(fmt)) return fail(FP8MI_ERR_ENUM, "fmt %d is not FP8MI_E4M3/FP8MI_E5M2", fmt);
  fp8mi_status s = check_scale_ring(nullptr, ring, hist_len);
  if (s != FP8MI_OK) return s;
  return from_hip(launch_ring_seed(ring, hist_len, amax, fmt, static_cast<hipStream_t>(stream)), "seed launch");
}

fp8mi_status fp8mi_stream_reference(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes,
                                    void* stream) {
  if (src_bytes < 0 || src_bytes % 16) return fail(FP8MI_ERR_ARG, "src_bytes %lld is not a multiple of 16",
                                                   (long long)src_bytes);
  if (dst_bytes != src_bytes && 2 * dst_bytes != src_bytes)
    return fail(FP8MI_ERR_ARG, "dst_bytes %lld must equal src_bytes %lld or its half", (long long)dst_bytes,
                (long long)src_bytes);
  if (src_bytes == 0) return FP8MI_OK;
  if (!src || !dst) return fail(FP8MI_ERR_NULL, "src or dst is NULL");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u)
    return fail(FP8MI_ERR_ARG, "src and dst must be 16-byte aligned");
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 < d0 + (uintptr_t)dst_bytes && d0 < s0 + (uintptr_t)src_bytes)
    return fail(FP8MI_ERR_ARG, "src and dst overlap");
  return from_hip(launch_stream(src, src_bytes, dst, dst_bytes, static_cast<hipStream_t>(stream)),
                  "stream reference launch");
}

const char* fp8mi_status_string(int s) {
  switch (s) {
    case FP8MI_OK: return "ok";
    case FP8MI_ERR_NULL: return "required pointer is NULL";
    case FP8MI_ERR_ENUM: return "enum value out of range";
    case FP8MI_ERR_SHAPE: return "invalid shape or leading dimension";
    case FP8MI_ERR_STRIDE: return "invalid batch stride";
    case FP8MI_ERR_UNSUPPORTED: return "unsupported layout or alignment";
    case FP8MI_ERR_HIP: return "HIP runtime error";
    case FP8MI_ERR_ARG: return "inconsistent arguments";
    default: return "unknown status";
  }
}

const char* fp8mi_last_error(void) { return g_err; }

const char* fp8mi_version(void) { return "fp8mi 0.1 gfx950"; }

}  // extern "C"
