/*
 * fp8mi -- FP8 per-tensor scaled quantize (delayed scaling with an in-kernel
 * amax history fold, or current scaling), per-tensor-scaled fp8 GEMM (fused
 * bias, bf16 or quantized fp8 output, layout tags) and the bias gradient, for
 * AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every pointer argument named "device" is a device (HBM) pointer;
 * every call is asynchronous on `stream` (a hipStream_t passed as void*;
 * NULL = the null stream) and allocates no memory.  The caller owns every
 * buffer.  Arguments are checked before anything is launched: a call that
 * returns a status other than FP8MI_OK has written nothing.  A HIP launch
 * failure returns FP8MI_ERR_HIP; fp8mi_last_error() then holds the HIP text.
 * Outputs must not overlap the inputs or each other (the results are then
 * undefined).  An extent -- rows x leading dimension x element bytes, or
 * batch x batch stride -- above 2^62 bytes is rejected with FP8MI_ERR_SHAPE.
 *
 * Citations are to the AstrAI commit-log pages (Gitea, ViperEkura/AstrAI);
 * "log:<path>" names the commit history page of that path.
 *
 * Number formats.  OCP FP8: E4M3 (E4M3FN: bias 7, no infinity, S.1111.111 is
 * NaN, largest 448) and E5M2 (bias 15, largest 57344).  Quantizing x with
 * per-tensor scale s stores enc(fl32(fl32(x) * s)): the input is widened
 * exactly to fp32, multiplied once in fp32 (round to nearest even, no flush
 * of subnormals) and encoded with saturating round-to-nearest-even (ties to
 * the even code; |v| >= fmt max and +-inf give +-max; NaN gives the format's
 * NaN code 0x7F with the input's sign; the sign of zero is kept).  Codes are
 * stored one byte per element, element j of a row at byte j (log:tests/extension,
 * the commit that fixes fp8 packing of four codes per 32-bit word).
 *
 * Amax.  max |fl32(x)| over the raw, unscaled input, NaN ignored
 * (log:csrc/kernels/fp8_mm.cu, commit 69f35c46e0).
 *
 * Ring (delayed scaling; log:tests/extension, the commits that pack
 * [history | scale | counter] into one device buffer and fold it in the
 * quantize kernel's last block).  A ring for a history of H amaxes is
 * FP8MI_RING_WORDS(H) = H + 4 + 1024 32-bit device words:
 *   [0, H)        amax history, fp32
 *   H             current scale, fp32 (the scale the next quantize call uses)
 *   H+1           next history slot, uint32 in [0, H)
 *   H+2           completion ticket, uint32, 0 at rest
 *   H+3           reserved, 0
 *   [H+4, H+1028) fold scratch: per-slot partial amax and counters on 32
 *                 separate 128-byte lines, all 0 at rest
 * The caller initialises it (history 0, slot 0, scale = a starting scale,
 * every other word 0) and may copy it to checkpoint / restore.  A fold of
 * amax a writes a into hist[slot], advances slot modulo H, and publishes
 * scale = fmt_max / max(hist) -- or 1.0 when that maximum is 0 or not finite
 * or the quotient is not a finite positive number.  After every call the
 * ticket and the scratch words are 0 again.  One ring may be used by at most
 * one call in flight at a time.
 */
#ifndef FP8MI_H
#define FP8MI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define FP8MI_API __attribute__((visibility("default")))
#else
#define FP8MI_API
#endif

typedef enum {
  FP8MI_OK = 0,
  FP8MI_ERR_NULL = 1,        /* a required pointer is NULL                       */
  FP8MI_ERR_ENUM = 2,        /* format / dtype value out of range                */
  FP8MI_ERR_SHAPE = 3,       /* negative size, ld smaller than the row, bad H    */
  FP8MI_ERR_STRIDE = 4,      /* batch strides that overlap written outputs       */
  FP8MI_ERR_UNSUPPORTED = 5, /* valid request outside the implemented fast path  */
  FP8MI_ERR_HIP = 6,         /* HIP runtime reported an error                     */
  FP8MI_ERR_ARG = 7          /* inconsistent optional arguments (scale vs ring)   */
} fp8mi_status;

typedef enum { FP8MI_E4M3 = 0, FP8MI_E5M2 = 1 } fp8mi_format;
typedef enum {
  FP8MI_F32 = 0,
  FP8MI_F16 = 1,
  FP8MI_BF16 = 2,
  FP8MI_FP8_E4M3 = 3, /* fp8 codes, one byte per element (bias / GEMM output of fp8_mm_ex) */
  FP8MI_FP8_E5M2 = 4
} fp8mi_dtype;

/* Largest history window a ring may have, and the ring size in words. */
#define FP8MI_MAX_HIST 4096
#define FP8MI_RING_SCRATCH_WORDS 1024
#define FP8MI_RING_WORDS(H) ((H) + 4 + FP8MI_RING_SCRATCH_WORDS)

/*
 * fp8_quantize -- per-tensor scaled cast of a [rows, cols] tensor to fp8 in
 * row or transposed layout (log:tests/extension, the commit that splits the
 * bindings into quantize(transposed) / quantize_dual with a layout enum;
 * log:csrc/kernels/fp8/quantize.cuh, the commit introducing the tiled
 * transposed quantize that handles odd widths and misaligned bases in-kernel).
 *
 *   x          device, element (i, j) at x[i * ld_x + j]; dtype x_dtype.
 *              Any base aligned to the element size (no 16-byte
 *              alignment needed); ld_x >= cols.
 *   fmt        FP8MI_E4M3 or FP8MI_E5M2.
 *   transposed 0: out[i * ld_out + j] = q(i, j), ld_out >= cols;
 *              1: out[j * ld_out + i] = q(i, j), ld_out >= rows.
 *              Bytes of `out` outside the rows x cols codes are not written.
 *   scale      device fp32 per-tensor scale, or NULL;
 *   ring       device ring of FP8MI_RING_WORDS(hist_len) words, or NULL.  Exactly one of
 *              scale / ring is given (else FP8MI_ERR_ARG).  With a ring the
 *              call uses the ring's current scale and its last workgroup folds
 *              this call's amax into the ring (the next scale is published
 *              on device; no host round trip).
 *   scale_inv_out  optional device fp32: 1 / (the scale this call used),
 *              i.e. the dequantisation multiplier for fp8_mm -- a snapshot
 *              taken before the fold replaces the ring's scale
 *              (log:tests/extension, the commit snapshotting sx/sw/sg).
 *   amax_out   optional device fp32: this call's raw amax.
 * rows * cols == 0 is a valid no-op for the codes; a ring still folds amax 0.
 */
FP8MI_API fp8mi_status fp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                          int fmt, int transposed, uint8_t* out, int64_t ld_out,
                          const float* scale, uint32_t* ring, int32_t hist_len,
                          float* scale_inv_out, float* amax_out, void* stream);

/*
 * fp8_quantize_dual -- one read of x, both layouts written: out_row (as
 * transposed = 0) and out_t (as transposed = 1); one amax, one fold
 * (log:csrc/kernels/fp8/quantize.cuh, the dual-layout "layout 2" of the
 * tiled quantize commit).  Arguments as fp8_quantize.
 */
FP8MI_API fp8mi_status fp8_quantize_dual(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                               int fmt, uint8_t* out_row, int64_t ld_row, uint8_t* out_t, int64_t ld_t,
                               const float* scale, uint32_t* ring, int32_t hist_len,
                               float* scale_inv_out, float* amax_out, void* stream);

/*
 * fp8_quantize_dynamic -- current (dynamic) scaling: the scale is measured
 * from x itself and used by the same call, with no ring (log:tests/extension,
 * the commit merging the delayed and dynamic recipes behind one `dynamic`
 * flag and the commit that allocates no scale rings on the dynamic path,
 * whose scales are measured inline).  s = fmt_max / amax(x) -- or 1.0 when
 * amax is 0 or not finite or the quotient is not a finite positive number,
 * exactly the scale a ring fold of amax(x) into an empty window publishes --
 * and x is quantized with s as in fp8_quantize.
 *   layout     0: row layout into out_row (ld_row >= cols); 1: transposed into
 *              out_t (ld_t >= rows); 2: both, from one read.  The pointer of an
 *              unused layout is ignored.
 *   scale_inv_out  optional device fp32: 1 / s, the dequantisation multiplier.
 *   amax_out   optional device fp32: amax(x).
 *   workspace  device scratch of at least FP8MI_DYNAMIC_WORKSPACE_BYTES bytes,
 *              4-byte aligned, owned by the caller, no initialisation (it
 *              carries per-workgroup partial maxima from the first launch to
 *              the second); calls in flight on one workspace race.
 * Other arguments as fp8_quantize.  Two launches on `stream`: an amax pass
 * over x, then the quantize pass, whose workgroups each reduce the partials to
 * s.  rows * cols == 0 gives amax 0 and s = 1.  A missing or short workspace
 * returns FP8MI_ERR_NULL / FP8MI_ERR_ARG before any launch.
 */
#define FP8MI_DYNAMIC_WORKSPACE_BYTES 4096
FP8MI_API fp8mi_status fp8_quantize_dynamic(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                            int fmt, int layout, uint8_t* out_row, int64_t ld_row, uint8_t* out_t,
                                            int64_t ld_t, float* scale_inv_out, float* amax_out, void* workspace,
                                            size_t workspace_bytes, void* stream);

/*
 * fp8_amax_fold -- the ring fold alone, for an amax already on the device
 * (e.g. one reduced over several devices): one tiny launch that performs
 * exactly the fold a ring-mode quantize performs in its last workgroup
 * (log:tests/extension, the commit testing the in-kernel fold against a host
 * reference).  ring: device, FP8MI_RING_WORDS(hist_len) words; amax:
 * device fp32.
 */
FP8MI_API fp8mi_status fp8_amax_fold(uint32_t* ring, int32_t hist_len, const float* amax, int fmt, void* stream);

/*
 * fp8_mm -- per-tensor-scaled fp8 GEMM, NT operands, bf16 output
 * (log:tests/extension: the commits fusing the fp32 bias ahead of a single
 * bf16 rounding, accepting 3-D operands through batch strides with stride-0
 * broadcast, and making the output always bf16; log:csrc/kernels/fp8_mm.cu,
 * commit 5244f1a8fc, per-tensor A/B scales applied inside the GEMM).
 *
 *   C[b,i,j] = bf16( fl32( sum_k dec(A[b,i,k]) * dec(B[b,j,k]) ) * fl32(sa * sb)
 *                    + bias[j] )      -- accumulated in fp32, one rounding.
 *   A(b,i,k) = a[b * stride_a + i * lda + k]   (fmt_a codes, device)
 *   B(b,j,k) = b[b * stride_b + j * ldb + k]   (fmt_b codes, device)
 *   C(b,i,j) = c[b * stride_c + i * ldc + j]   (bf16, device)
 *   stride_a / stride_b may be 0 (one operand broadcast over the batch).
 *   a_scale_inv, b_scale_inv: device fp32 dequantisation multipliers
 *   (e.g. scale_inv_out of the quantize calls), NULL meaning 1.0.
 *   bias: device [N] of bias_dtype (FP8MI_F32 / FP8MI_F16 / FP8MI_BF16), one
 *   vector shared by every row and batch; NULL for no bias.
 * Requirements: a, b 16-byte aligned; lda, ldb, K multiples of 16 (else
 * FP8MI_ERR_UNSUPPORTED); lda, ldb >= K; ldc >= N; c 2-byte aligned; with
 * batch > 1, stride_c >= M * ldc.  M, N or batch 0: no-op.  K == 0 writes
 * bf16(bias) (or zeros).  Launch-grid limits: ceil(M / 64) <= 65535,
 * batch <= 65535 and ceil(M / 64) * ceil(N / 64) < 2^29 (else
 * FP8MI_ERR_UNSUPPORTED).
 */
FP8MI_API fp8mi_status fp8_mm(const uint8_t* a, int fmt_a, int64_t lda, int64_t stride_a,
                    const uint8_t* b, int fmt_b, int64_t ldb, int64_t stride_b,
                    int64_t M, int64_t N, int64_t K, int64_t batch,
                    const float* a_scale_inv, const float* b_scale_inv,
                    const void* bias, int bias_dtype,
                    void* c, int64_t ldc, int64_t stride_c, void* stream);

/*
 * fp8_mm_ex -- fp8_mm with an fp8-stored bias and an optional quantizing
 * epilogue (FP8-in / FP8-out GEMM; log:tests/extension, the commit adding the
 * FP8-in/FP8-out GEMM op and the commit giving the bias a bias_scale slot:
 * no scale = a raw bias, a scale = fp8 storage dequantized in the epilogue
 * after the operand scaling and before any output quantization).
 *   y[b,i,j] = fl32( sum_k dec(A) dec(B) ) * fl32(sa * sb) + bias_j   (fp32)
 *   bias_j     bias_dtype FP8MI_F32 / F16 / BF16: the value, widened exactly
 *              (bias_scale must be NULL); FP8MI_FP8_E4M3 / E5M2: fl32(dec(code)
 *              * *bias_scale), bias_scale a device fp32 (required).
 *   c_dtype    FP8MI_BF16: C = bf16(y), exactly fp8_mm (c_scale, c_ring,
 *              c_scale_inv_out and c_amax_out must be NULL).
 *              FP8MI_FP8_E4M3 / E5M2: C holds codes enc(fl32(y * s_c)), one byte
 *              per element, C(b,i,j) at c[b * stride_c + i * ldc + j] (element
 *              strides); the output is quantized like an fp32 tensor by
 *              fp8_quantize: s_c = *c_scale, or the ring c_ring's current scale
 *              (exactly one of the two; ring layout and fold as fp8_quantize),
 *              amax = max |y| over every output of every batch (NaN ignored),
 *              one fold of it into the ring, c_scale_inv_out = 1 / s_c and
 *              c_amax_out = amax (both optional).  Operand extents must stay
 *              below 2^31 bytes (else FP8MI_ERR_UNSUPPORTED).
 *   layout     0, or FP8MI_A_KM and / or FP8MI_B_KM: an operand given K-major
 *              (e.g. a transposed view of a row-major [K, M] array), read
 *              without a transposed copy (the pages' layout tags from .t()
 *              views: log:tests/extension, the commit taking transposed and
 *              3-D operands into the GEMM).  A K-major A is a [K, lda] array
 *              of K full rows (K * lda readable bytes per batch, the last
 *              row's padding included) with lda >= M (B: [K, ldb], ldb >= N),
 *              lda % 16 == 0 and extents below 2^31 bytes (else
 *              FP8MI_ERR_UNSUPPORTED), with either output type; the result
 *              (bf16 values, or fp8 codes, amax and ring words) is that of the
 *              same operands in NT form, bit for bit.
 * Other arguments and requirements as fp8_mm.  M, N or batch 0 writes no
 * codes; an fp8 output then still folds amax 0 into its ring (or writes
 * 1 / s_c and amax 0).  y is fp32, so its accumulation error is that of
 * fp8_mm before the bf16 rounding; an output near a code boundary may take
 * the neighbouring code.
 */
#define FP8MI_A_KM 1 /* layout tag: A stored K-major, A(b,i,k) = a[b * stride_a + k * lda + i] */
#define FP8MI_B_KM 2 /* layout tag: B stored K-major, B(b,j,k) = b[b * stride_b + k * ldb + j] */
FP8MI_API fp8mi_status fp8_mm_ex(const uint8_t* a, int fmt_a, int64_t lda, int64_t stride_a,
                                 const uint8_t* b, int fmt_b, int64_t ldb, int64_t stride_b,
                                 int64_t M, int64_t N, int64_t K, int64_t batch, int layout,
                                 const float* a_scale_inv, const float* b_scale_inv,
                                 const void* bias, int bias_dtype, const float* bias_scale,
                                 void* c, int c_dtype, int64_t ldc, int64_t stride_c,
                                 const float* c_scale, uint32_t* c_ring, int32_t c_hist_len,
                                 float* c_scale_inv_out, float* c_amax_out, void* stream);

/*
 * fp8_quantize_dual_bias_grad -- fp8_quantize_dual of an output gradient
 * plus its bias gradient from the same read: the codes, scale_inv and ring
 * update are exactly those of fp8_quantize_dual, and bias_grad_out[j] is the
 * sum of the raw dy[i, j] over all rows (the pages reduce grad_b over the
 * leading dimensions of the gradient before any quantization:
 * log:tests/extension, the commit fixing the 3-D backward and the commit
 * forcing gradients to bf16), accumulated in fp64 in a fixed order and
 * rounded once to bf16 -- within rounding of fp8_bias_grad, whose summation
 * order differs.
 *   x            the gradient, FP8MI_BF16 or FP8MI_F16 (FP8MI_F32 returns
 *                FP8MI_ERR_UNSUPPORTED); other arguments as fp8_quantize_dual.
 *   bias_grad_out  device bf16 [cols].
 *   workspace    as fp8_bias_grad: fp8_bias_grad_workspace_bytes(rows, cols)
 *                bytes, 8-byte aligned, caller-owned, no initialisation.
 * Two launches (the dual quantize, then a small finalize) on `stream`.
 */
FP8MI_API fp8mi_status fp8_quantize_dual_bias_grad(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                                   int64_t ld_x, int fmt, uint8_t* out_row, int64_t ld_row,
                                                   uint8_t* out_t, int64_t ld_t, const float* scale, uint32_t* ring,
                                                   int32_t hist_len, float* scale_inv_out, float* amax_out,
                                                   void* bias_grad_out, void* workspace, size_t workspace_bytes,
                                                   void* stream);

/*
 * fp8_quantize_dual_bias_grad_noalloc -- fp8_quantize_dual_bias_grad for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving or training loops, harnesses that forbid allocation): the
 * same arguments without the workspace, the same results bit for bit.  The
 * per-tile column sums go to a scratch array the library owns, one per GPU,
 * FP8MI_NOALLOC_SCRATCH_BYTES bytes, held from the first call on that GPU
 * until the process ends.  The call allocates nothing (no hipMalloc, no
 * allocating library routine).  A gradient whose sums need more than the
 * array, fp8_bias_grad_workspace_bytes(rows, cols) >
 * FP8MI_NOALLOC_SCRATCH_BYTES (8 MiB: ceil(rows / 128) * cols <= 1048576,
 * e.g. 8192 x 6912 uses 3.5 MB), returns FP8MI_ERR_UNSUPPORTED before any
 * launch.  Every call on one GPU shares its array, and nothing in it needs
 * clearing (each call writes every sum it reads): calls that overlap on one
 * GPU (different streams, or host threads without ordering) race.
 */
#define FP8MI_NOALLOC_SCRATCH_BYTES (8 * 1024 * 1024)
FP8MI_API fp8mi_status fp8_quantize_dual_bias_grad_noalloc(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                                           int64_t ld_x, int fmt, uint8_t* out_row, int64_t ld_row,
                                                           uint8_t* out_t, int64_t ld_t, const float* scale,
                                                           uint32_t* ring, int32_t hist_len, float* scale_inv_out,
                                                           float* amax_out, void* bias_grad_out, void* stream);

/*
 * fp8_bias_grad -- bias gradient of an fp8 linear layer: out[j] = the sum of
 * dy[i, j] over all rows i (every leading dimension flattened into rows),
 * accumulated in fp64 in a fixed order and rounded once to bf16
 * (log:tests/extension, the commit reducing grad_b over leading dims; the
 * commit forcing gradients to bf16).
 *   dy         device, element (i, j) at dy[i * ld + j], dy_dtype FP8MI_BF16
 *              or FP8MI_F16 (FP8MI_F32 returns FP8MI_ERR_UNSUPPORTED);
 *              ld >= cols.
 *   out        device bf16 [cols].
 *   workspace  device scratch owned by the caller, 8-byte aligned, at least
 *              fp8_bias_grad_workspace_bytes(rows, cols) bytes (NULL allowed
 *              when that is 0).  Its contents are overwritten and need no
 *              initialisation; calls in flight on the same workspace race.
 * rows == 0 writes zeros; cols == 0 is a no-op.  A workspace that is missing
 * or too small returns FP8MI_ERR_NULL / FP8MI_ERR_ARG before any launch.
 */
FP8MI_API fp8mi_status fp8_bias_grad(const void* dy, int dy_dtype, int64_t rows, int64_t cols, int64_t ld,
                                     void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8_bias_grad_workspace_bytes -- device workspace fp8_bias_grad needs for a
 * [rows, cols] gradient (per-chunk fp64 column sums); 0 when rows or cols is
 * not positive.  Pure host function.
 */
FP8MI_API size_t fp8_bias_grad_workspace_bytes(int64_t rows, int64_t cols);

/*
 * fp8_ring_seed -- (re)initialise a ring on the device: history, ticket and
 * scratch set to 0, slot 0, and current scale = the scale a fold of *amax
 * into an empty window would publish (fmt_max / amax, or 1.0 when amax is 0
 * or not finite).  This is the ring's seed step (log:tests/extension, the
 * commit giving the scale ring update / seed operations); *amax is typically
 * the amax_out of a quantize of the first tensor.  ring: device,
 * FP8MI_RING_WORDS(hist_len) words; amax: device fp32.
 */
FP8MI_API fp8mi_status fp8_ring_seed(uint32_t* ring, int32_t hist_len, const float* amax, int fmt, void* stream);

/*
 * fp8mi_stream_reference -- measurement aid, not part of the method: reads
 * src_bytes of src and writes dst_bytes of dst with the row quantize's access
 * shape and no arithmetic, so its time is the practical HBM ceiling for a
 * quantize moving the same bytes (row / transposed: dst_bytes = src_bytes / 2
 * for a 16-bit input; dual: dst_bytes = src_bytes).  dst receives bytes of src
 * (the top byte of every 16-bit pair, or src itself).  src and dst: device,
 * 16-byte aligned, not overlapping; src_bytes a multiple of 16; dst_bytes
 * equal to src_bytes or to its half, else FP8MI_ERR_ARG.  One launch.
 */
FP8MI_API fp8mi_status fp8mi_stream_reference(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes,
                                              void* stream);

/* Static text of a status code. */
FP8MI_API const char* fp8mi_status_string(int status);
/* Thread-local detail of the last non-OK status returned on this thread. */
FP8MI_API const char* fp8mi_last_error(void);
/* Library version, e.g. "fp8mi 0.1 gfx950". */
FP8MI_API const char* fp8mi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FP8MI_H */
