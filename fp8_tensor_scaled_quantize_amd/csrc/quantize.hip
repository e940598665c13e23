// Per-tensor scaled fp8 quantize for gfx950: row, transposed and dual layouts,
// raw-value amax and the in-kernel ring fold.
//
// log:csrc/kernels/fp8/quantize.cuh (the tiled transposed quantize commit):
// one tiled kernel serves the transposed layout ("layout 1") and the dual
// layout ("layout 2"), handling odd widths and misaligned bases inside the
// kernel; the elementwise (row) quantize is a separate streaming kernel.
// log:tests/extension (the in-kernel ring fold commit): the history update
// and the next scale are computed inside the quantize launch, by whichever
// workgroup completes last, instead of by separate kernels.
// log:csrc/kernels/fp8_mm.cu, commit 69f35c46e0: amax is taken from the raw
// input, never from the scaled or encoded values.
//
// MI355X shape of the kernels (not the pages' sm_89 one):
//  * quantize_flat: contiguous row layout; each wave moves 64 x 16-byte loads
//    per step (one contiguous 1 KiB segment per load instruction) and writes
//    one contiguous segment of codes per store instruction.  One-shot
//    workgroups while the tensor fits 8 per CU, else persistent ones with the
//    next group of steps loading while one is encoded.
//  * quantize_tiled / quantize_tiled_pf: 128-row x 64-column tiles, 256
//    threads.  Each thread loads a 4-row x 8-column micro block (16-byte
//    loads, realigned in registers when a row segment does not start on 16
//    bytes), so the row-layout codes leave straight from registers and the
//    transposed codes need only a 4x4 byte transpose in registers plus one
//    8 KiB LDS pass, after which every lane stores 16 contiguous bytes of a
//    transposed row (128-byte segments per 8 lanes).  One tile per workgroup
//    (quantize_tiled) or persistent workgroups with the next tile loading
//    while one is encoded (quantize_tiled_pf), by the same size rule.
//  * amax: wave and workgroup max on the raw bit patterns, then the ring's
//    slot protocol (the last workgroup folds) or one device-scope atomic max
//    into the caller's word.
//  * current scaling: amax_partials writes one partial max per workgroup to
//    the caller's workspace; the kernels above, instantiated with DYN, read
//    them all and derive the scale in every wave (no atomics).
#include "fp8mi_device.h"
#include "fp8mi_internal.h"

namespace fp8mi {

struct QuantArgs {
  const void* x;
  int64_t rows, cols, ld_x;
  uint8_t* out_row;
  int64_t ld_row;
  uint8_t* out_t;
  int64_t ld_t;
  const float* scale;   // explicit scale, or null with a ring
  uint32_t* ring;       // ring buffer, or null
  int H;
  float* scale_inv_out;
  float* amax_out;
  double* bias_ws;      // dual with bias gradient: fp64 column sums per 128-row tile, [tile row][col]
  const uint32_t* parts;  // current scaling: per-workgroup amax partials (fp32 bits), or null
  int nparts;
};

// Max over the current-scaling partials (n >= 1), computed by one whole wave;
// the result is valid in every lane.  The partials are non-negative fp32 bit
// patterns, which order like their values, so an integer max is exact and
// independent of order.
__device__ __forceinline__ float parts_max(const uint32_t* parts, int n) {
  constexpr int kLoads = 16;  // 1024 partials (a full workspace) in one batch
  const int lane = threadIdx.x & 63;
  uint32_t m = 0;
  for (int base = 0; base < n; base += 64 * kLoads) {
    uint32_t v[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int i = base + 64 * j + lane;
      v[j] = parts[i < n ? i : n - 1];  // a repeated partial leaves the max unchanged
    }
#pragma unroll
    for (int j = 0; j < kLoads; ++j) m = max(m, v[j]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  return __uint_as_float(m);
}

// Shared ending of every quantize workgroup.
template <int FMT, int NT, bool DYN>
__device__ __forceinline__ void quant_block_done(const QuantArgs& p, float thread_amax, float s, float* red) {
  if constexpr (DYN) {
    // current scaling: amax was measured by the partials pass; no atomics
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 64) {
      const float a = parts_max(p.parts, p.nparts);
      if (threadIdx.x == 0) {
        if (p.amax_out) *p.amax_out = a;
        if (p.scale_inv_out) *p.scale_inv_out = 1.0f / s;
      }
    }
    return;
  }
  const float bmax = block_max<NT>(thread_amax, red);
  if (p.ring) {
    ring_block_done<FMT>(p.ring, p.H, bmax, s, p.scale_inv_out, p.amax_out, reinterpret_cast<uint32_t*>(red));
  } else if (threadIdx.x == 0) {
    if (p.amax_out) publish_max(reinterpret_cast<uint32_t*>(p.amax_out), bmax);
    if (p.scale_inv_out && blockIdx.x == 0 && blockIdx.y == 0) *p.scale_inv_out = 1.0f / s;
  }
}

// Running max of |x| over raw 16-byte loads, on the bit patterns: for each
// input type the bits of |x| order exactly like the magnitudes, and NaNs sort
// above infinity, so one integer max (packed 16-bit for bf16 / fp16) yields
// both the amax and whether a NaN was seen.
template <int DT> struct AbsMax;
template <> struct AbsMax<kBF16> {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  us2 m = {0, 0};
  __device__ __forceinline__ void add(const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, w[e] & 0x7FFF7FFFu));
  }
  __device__ __forceinline__ uint32_t top() const { return m[0] > m[1] ? m[0] : m[1]; }
  __device__ __forceinline__ bool has_nan() const { return top() > 0x7F80u; }
  __device__ __forceinline__ float value() const { return bf16_to_f32(top()); }
};
template <> struct AbsMax<kF16> {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  us2 m = {0, 0};
  __device__ __forceinline__ void add(const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, w[e] & 0x7FFF7FFFu));
  }
  __device__ __forceinline__ uint32_t top() const { return m[0] > m[1] ? m[0] : m[1]; }
  __device__ __forceinline__ bool has_nan() const { return top() > 0x7C00u; }
  __device__ __forceinline__ float value() const { return f16_to_f32(top()); }
};
template <> struct AbsMax<kF32> {
  uint32_t m = 0;
  __device__ __forceinline__ void add(const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) m = max(m, w[e] & 0x7FFFFFFFu);
  }
  __device__ __forceinline__ bool has_nan() const { return m > 0x7F800000u; }
  __device__ __forceinline__ float value() const { return __uint_as_float(m); }
};

// max |v| over the non-NaN values.  The fast loops use v_max_f32, which is
// not NaN-free when an operand is a signalling NaN (it returns a quiet NaN),
// so a chunk that holds any NaN recomputes its amax here.
template <int N> __device__ __forceinline__ float nan_free_absmax(const float* f) {
  float m = 0.0f;
#pragma unroll
  for (int e = 0; e < N; ++e)
    if (f[e] == f[e]) m = fmaxf(m, fabsf(f[e]));
  return m;
}

// The scale this call quantizes with: measured from the partials (DYN,
// current scaling), else the ring's current scale (delayed scaling) or the
// caller's.  DYN is a template parameter so that the delayed-scaling kernels
// carry none of the partials code (it would cost them registers).
// 16 * NLD bytes from src (element-aligned, any 16-byte misalignment) as NLD
// uint4.  Global vector loads on CDNA need only dword alignment, so the data
// comes from dword-aligned 16-byte loads at src rounded down to 4 bytes (plus
// one more dword when that drops 2 bytes, as a 16-bit element start can),
// shifted by v_alignbyte.  Every load holds at least one requested byte and
// none lies beyond the last one plus 3, so all stay on pages the tensor
// occupies.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
template <int NLD> __device__ __forceinline__ void load16_any(const char* src, uint4 (&out)[NLD]) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(src);
  if ((a & 15u) == 0) {
#pragma unroll
    for (int c = 0; c < NLD; ++c) out[c] = reinterpret_cast<const uint4*>(src)[c];
    return;
  }
  const uint32_t sb = (uint32_t)(a & 3u);  // 0 or 2 (elements are 2 or 4 bytes)
  const char* a4 = src - sb;
  uint32_t w[4 * NLD + 1];
#pragma unroll
  for (int c = 0; c < NLD; ++c) {
    const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(a4 + 16 * c);
    w[4 * c] = v.x; w[4 * c + 1] = v.y; w[4 * c + 2] = v.z; w[4 * c + 3] = v.w;
  }
  w[4 * NLD] = sb ? *reinterpret_cast<const uint32_t*>(a4 + 16 * NLD) : 0u;
#pragma unroll
  for (int c = 0; c < NLD; ++c) {
    out[c].x = __builtin_amdgcn_alignbyte(w[4 * c + 1], w[4 * c], sb);
    out[c].y = __builtin_amdgcn_alignbyte(w[4 * c + 2], w[4 * c + 1], sb);
    out[c].z = __builtin_amdgcn_alignbyte(w[4 * c + 3], w[4 * c + 2], sb);
    out[c].w = __builtin_amdgcn_alignbyte(w[4 * c + 4], w[4 * c + 3], sb);
  }
}

template <int FMT, bool DYN> __device__ __forceinline__ float read_scale(const QuantArgs& p) {
  if constexpr (DYN) return scale_from_max<FMT>(parts_max(p.parts, p.nparts));
  else return p.ring ? __uint_as_float(p.ring[p.H]) : *p.scale;
}

// ===========================================================================
// Row layout, contiguous input and output (ld == cols), 16-byte aligned bases.
// A "wave step" covers 64 lanes x 16 elements; a lane holds NL 16-byte loads
// whose element offsets are (j * 64 + lane) * EPL within the step.
// ===========================================================================
constexpr int kFlatThreads = 256;
constexpr int kFlatElemsPerThread = 16;
constexpr int kFlatWaveStep = 64 * kFlatElemsPerThread;                   // 1024 elements
constexpr int kFlatBlockStep = kFlatThreads * kFlatElemsPerThread;      // 4096 elements
constexpr int kFlatUnroll = 2;                                          // block steps in flight per lane

// One lane's 16 elements of a wave step as fp32 values.
template <int DT, int NL>
__device__ __forceinline__ void flat_widen(const uint4 (&v)[NL], float (&f)[kFlatElemsPerThread]) {
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
    if constexpr (DT == kF32) {
#pragma unroll
      for (int e = 0; e < 4; ++e) f[j * 4 + e] = __uint_as_float(w[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) widen2<DT>(w[e], f[j * 8 + 2 * e], f[j * 8 + 2 * e + 1]);
    }
  }
}

// Max |x| over one lane's 16 elements of a wave step, NaNs skipped -- the
// value flat_encode_store returns for the same loads.
template <int DT, int NL> __device__ __forceinline__ float flat_absmax(const uint4 (&v)[NL]) {
  AbsMax<DT> am;
#pragma unroll
  for (int j = 0; j < NL; ++j) am.add(v[j]);
  if (!am.has_nan()) return am.value();
  float f[kFlatElemsPerThread];
  flat_widen<DT, NL>(v, f);
  return nan_free_absmax<kFlatElemsPerThread>(f);
}

// Encode one lane's 16 elements of a wave step (already loaded) and store the codes.
template <int DT, int FMT, int NL, int EPL>
__device__ __forceinline__ float flat_encode_store(const uint4 (&v)[NL], uint8_t* out_w0, int lane, float s,
                                                   bool sreg) {
  float f[kFlatElemsPerThread];
  flat_widen<DT, NL>(v, f);
  AbsMax<DT> am;
#pragma unroll
  for (int j = 0; j < NL; ++j) am.add(v[j]);
  const bool nan = am.has_nan();
  const float camax = nan ? nan_free_absmax<kFlatElemsPerThread>(f) : am.value();
  uint32_t code[kFlatElemsPerThread / 4];
  if (!nan && sreg && camax * fabsf(s) <= FmtTraits<FMT>::kMax) {
    // no clamp needed: fl32(|x| |s|) <= fl32(camax |s|) (monotonic rounding)
#pragma unroll
    for (int q = 0; q < kFlatElemsPerThread / 4; ++q)
      code[q] = cvt4_inrange<FMT>(f[4 * q] * s, f[4 * q + 1] * s, f[4 * q + 2] * s, f[4 * q + 3] * s);
  } else if (!nan && sreg) {
#pragma unroll
    for (int q = 0; q < kFlatElemsPerThread / 4; ++q)
      code[q] = cvt4<FMT>(f[4 * q] * s, f[4 * q + 1] * s, f[4 * q + 2] * s, f[4 * q + 3] * s);
  } else {
#pragma unroll
    for (int q = 0; q < kFlatElemsPerThread / 4; ++q)
      code[q] = enc4_exact<FMT>(f[4 * q] * s, f[4 * q + 1] * s, f[4 * q + 2] * s, f[4 * q + 3] * s);
  }
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    uint8_t* o = out_w0 + (int64_t)(j * 64 + lane) * EPL;
    if constexpr (EPL == 8) *reinterpret_cast<uint2*>(o) = make_uint2(code[2 * j], code[2 * j + 1]);
    else *reinterpret_cast<uint32_t*>(o) = code[j];
  }
  return camax;
}

// Each block handles `steps_per_block` consecutive block steps in groups of
// kFlatUnroll.  With PF the groups are software-pipelined over two register
// buffers (the loads of group g + 1 in flight while group g is encoded), for
// persistent grids over large tensors; without it a block holds one group
// at a time, which keeps registers low and occupancy high for the grids that
// give every workgroup a single group.
template <int DT, int FMT, bool PF, bool DYN>
__global__ void __launch_bounds__(kFlatThreads) quantize_flat(QuantArgs p, int64_t n, int64_t steps_per_block) {
  __shared__ float red[kFlatThreads / 64];
  constexpr int EB = In<DT>::kBytes;
  constexpr int EPL = 16 / EB;                   // elements per 16-byte load
  constexpr int NL = kFlatElemsPerThread / EPL;  // loads per lane per step
  constexpr int U = kFlatUnroll;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  float amax = 0.0f;
  const char* xb = static_cast<const char*>(p.x);
  const int64_t first = (int64_t)blockIdx.x * steps_per_block;
  const int64_t total_steps = (n + kFlatBlockStep - 1) / kFlatBlockStep;
  const int64_t last = first + steps_per_block < total_steps ? first + steps_per_block : total_steps;
  // groups of U steps that lie wholly inside the tensor
  const int64_t full_end = last < n / kFlatBlockStep ? last : n / kFlatBlockStep;
  const int64_t ng = full_end > first ? (full_end - first) / U : 0;
  auto load_group = [&](uint4 (&v)[U][NL], int64_t g0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t w0 = (g0 + u) * kFlatBlockStep + (int64_t)wid * kFlatWaveStep;
#pragma unroll
      for (int j = 0; j < NL; ++j)
        v[u][j] = *reinterpret_cast<const uint4*>(xb + (w0 + (int64_t)(j * 64 + lane) * EPL) * EB);
    }
  };
  uint4 va[U][NL];
  if (ng > 0) load_group(va, first);
  // the scale is read after the first loads are out (it does not gate them)
  const float s = read_scale<FMT, DYN>(p);
  const bool sreg = scale_regular(s);
  auto encode_group = [&](const uint4 (&v)[U][NL], int64_t g0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t w0 = (g0 + u) * kFlatBlockStep + (int64_t)wid * kFlatWaveStep;
      amax = fmaxf(amax, flat_encode_store<DT, FMT, NL, EPL>(v[u], p.out_row + w0, lane, s, sreg));
    }
  };
  if constexpr (!PF && !DYN) {
    // A ring-mode workgroup whose whole share is one group knows its amax
    // before it stores anything: it publishes first, so the slot atomic's
    // round trip overlaps the encoding and the stores.
    if (p.ring && ng == 1 && first + U == last) {
      float a = 0.0f;
#pragma unroll
      for (int u = 0; u < U; ++u) a = fmaxf(a, flat_absmax<DT, NL>(va[u]));
      const float bmax = block_max<kFlatThreads>(a, red);
      uint32_t pub = __builtin_nondeterministic_value(0u);  // read by thread 0 only
      if (threadIdx.x == 0) pub = ring_publish(p.ring, p.H, bmax);
      encode_group(va, first);
      ring_block_finish<FMT>(p.ring, p.H, pub, s, p.scale_inv_out, p.amax_out, reinterpret_cast<uint32_t*>(red));
      return;
    }
  }
  int64_t g = 0;
  if constexpr (PF) {
    uint4 vb[U][NL];
    for (; g + 2 <= ng; g += 2) {
      load_group(vb, first + (g + 1) * U);
      encode_group(va, first + g * U);
      if (g + 2 < ng) load_group(va, first + (g + 2) * U);
      encode_group(vb, first + (g + 1) * U);
    }
  } else {
    for (; g + 1 < ng; ++g) {
      encode_group(va, first + g * U);
      load_group(va, first + (g + 1) * U);
    }
  }
  if (g < ng) encode_group(va, first + g * U);
  int64_t st = first + ng * U;
  for (; st < last; ++st) {
    const int64_t w0 = st * kFlatBlockStep + (int64_t)wid * kFlatWaveStep;
    if (w0 + kFlatWaveStep <= n) {
      uint4 v[NL];
#pragma unroll
      for (int j = 0; j < NL; ++j)
        v[j] = *reinterpret_cast<const uint4*>(xb + (w0 + (int64_t)(j * 64 + lane) * EPL) * EB);
      amax = fmaxf(amax, flat_encode_store<DT, FMT, NL, EPL>(v, p.out_row + w0, lane, s, sreg));
    } else if (w0 < n) {
      // ragged end of the tensor: element by element, same lane mapping
#pragma unroll
      for (int j = 0; j < NL; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const int64_t idx = w0 + (int64_t)(j * 64 + lane) * EPL + e;
          if (idx < n) {
            const float xv = load1<DT>(p.x, idx);
            if (xv == xv) amax = fmaxf(amax, fabsf(xv));
            p.out_row[idx] = (uint8_t)enc_exact<FMT>(xv * s);
          }
        }
      }
    }
  }
  quant_block_done<FMT, kFlatThreads, DYN>(p, amax, s, red);
}

// ===========================================================================
// Tiled kernel: transposed, dual, and row layout for strided / misaligned /
// odd-width inputs.  Tile = 128 rows x 64 columns, 256 threads.
// Thread t: column group cg = t % 8 (columns 8cg..8cg+7), row group
// rg = t / 8 (rows 4rg..4rg+3).
// LDS (transposed codes): 64 columns x 32 words; word w of column c holds
// rows 4w..4w+3 and sits at c*32 + (w ^ (8 * ((c / 8) & 3))).
// ===========================================================================
constexpr int kTileR = 128, kTileC = 64, kTileThreads = 256;
enum Mode : int { kRow = 0, kTrans = 1, kDual = 2 };

// Bias-gradient partials in LDS: row group g (32 of them, 4 rows each) and
// column c at g * 64 + (c ^ (g & 7)).  A write instruction (fixed column
// offset e, lanes over 8 row groups x 8 column groups) then spreads over 32
// distinct 8-byte bank pairs, and a read (one row group, 64 consecutive
// columns) stays a permutation of one 512-byte row.
__device__ __forceinline__ int bg_index(int g, int c) { return g * 64 + (c ^ (g & 7)); }

__device__ __forceinline__ int lds_t_index(int c, int w) { return c * 32 + (w ^ (8 * ((c >> 3) & 3))); }

// Tile origin (row, column) of a tile index: 32-bit division whenever the
// tile count fits (every tensor a GPU can hold), 64-bit otherwise; the
// branch is uniform across the workgroup.
__device__ __forceinline__ void tile_origin(int64_t tile, int64_t tiles_c, int64_t ntiles, int64_t& r0,
                                            int64_t& c0) {
  if (ntiles <= 0xFFFFFFFFll) {
    const uint32_t t = (uint32_t)tile, tc = (uint32_t)tiles_c;
    const uint32_t q = t / tc;
    r0 = (int64_t)q * kTileR;
    c0 = (int64_t)(t - q * tc) * kTileC;
  } else {
    r0 = (tile / tiles_c) * kTileR;
    c0 = (tile % tiles_c) * kTileC;
  }
}

// One-shot dual grids: workgroups are dealt to the 8 XCDs round-robin, and a
// tile's row codes fill one half of each 128-byte line, the column
// neighbour's tile the other.  Workgroups b and b + 8 (the same XCD, launched
// one after the other) take tiles 2k and 2k + 1 of each group of 16, so the two
// halves of a line meet in one L2 and leave it together; the XCDs still take
// neighbouring pairs in turn.  (Measured at bf16 8192 x 1536, alternating
// libraries on one box: dual 14.5 -> 14.25 us with a ring, 12.4 -> 12.1 us with
// a scale; giving each XCD one contiguous range of tiles instead gained about
// as much for the dual and slowed the transposed layout by 6-9%.)
__device__ __forceinline__ uint32_t dual_pair_block(uint32_t b, uint32_t nb) {
  const uint32_t full = nb / 16u * 16u;
  if (b >= full) return b;
  const uint32_t r = b % 16u;
  return b - r + 2u * (r % 8u) + r / 8u;
}

// 4 x 4 byte transpose: words a, b, c, d hold 4 consecutive codes of rows 0..3;
// col[k] receives byte k of each, row 0 in its low byte.  Two stages of
// v_perm_b32 (byte k of the result picks byte sel_k of {hi, lo}, 0-3 from lo,
// 4-7 from hi): interleave row pairs, then take the matching halves.
__device__ __forceinline__ void transpose4x4_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t (&col)[4]) {
  const uint32_t ab_lo = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
  const uint32_t ab_hi = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
  const uint32_t cd_lo = __builtin_amdgcn_perm(d, c, 0x05010400u);  // c0 d0 c1 d1
  const uint32_t cd_hi = __builtin_amdgcn_perm(d, c, 0x07030602u);  // c2 d2 c3 d3
  col[0] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);         // a0 b0 c0 d0
  col[1] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);         // a1 b1 c1 d1
  col[2] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);         // a2 b2 c2 d2
  col[3] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);         // a3 b3 c3 d3
}

// One-shot form: each workgroup loads, encodes and stores its tiles in turn
// (launched with one tile per workgroup; low registers, high occupancy).
// AL: every tile lies inside the tensor and every row of x, the row codes
// and the transposed codes starts 16 / 8 / 16 bytes aligned (checked by the
// launcher), so no bounds or alignment tests and no element-wise fallbacks
// are compiled -- which also lets the compiler count the stores exactly.
template <int DT, int FMT, int MODE, bool BG, bool DYN, bool AL>
__global__ void __launch_bounds__(kTileThreads) quantize_tiled(QuantArgs p, int64_t tiles_c, int64_t ntiles,
                                                                int64_t tiles_per_block) {
  __shared__ float red[kTileThreads / 64];
  __shared__ __align__(16) uint32_t lds_t[(MODE == kRow) ? 1 : kTileC * 32];
  __shared__ double bg_part[BG ? kTileR / 4 * kTileC : 1];  // [row group][column], swizzled
  constexpr int EB = In<DT>::kBytes;
  const float s = read_scale<FMT, DYN>(p);
  const bool sreg = scale_regular(s);
  const int t = threadIdx.x, cg = t & 7, rg = t >> 3;
  float amax = 0.0f;
  const char* xb = static_cast<const char*>(p.x);
  const uint32_t bid = MODE == kDual ? dual_pair_block(blockIdx.x, gridDim.x) : blockIdx.x;
  const int64_t t_first = (int64_t)bid * tiles_per_block;
  const int64_t t_last = t_first + tiles_per_block < ntiles ? t_first + tiles_per_block : ntiles;
  const bool x_rows16 = (reinterpret_cast<uintptr_t>(p.x) & 15u) == 0 && ((p.ld_x * EB) & 15) == 0;
  // A ring-mode workgroup of one transposed / dual tile publishes its amax
  // before any of its codes are stored, so the slot atomic's round trip
  // overlaps the stores: the general path as soon as its values are loaded
  // (before encoding), the transposed fast path once the tile is encoded (a
  // separate amax pass ahead of its row-by-row encode was slower).
  const bool early = MODE != kRow && !DYN && p.ring != nullptr && t_last - t_first == 1;
  uint32_t pub = __builtin_nondeterministic_value(0u);  // read by thread 0 only
  bool pubd = false;  // published already (the general path does it before encoding)
  for (int64_t tile = t_first; tile < t_last; ++tile) {
    int64_t r0, c0;
    tile_origin(tile, tiles_c, ntiles, r0, c0);
    const int64_t cc = c0 + 8 * cg;  // this thread's first column
    uint32_t rw[4][2];  // row words: rw[i][h] = codes of row i, columns 4h..4h+3
    float f[4][8];      // the values (general path; the bias gradient reads them)
    if (MODE == kTrans && (AL || (x_rows16 && r0 + kTileR <= p.rows && c0 + kTileC <= p.cols))) {
      // transposed output, tile inside the tensor, rows on 16 bytes: the four
      // rows' loads go out back to back, then each row is encoded on its own
      // (its own NaN and in-range tests, which give the same codes as the
      // tile-wide tests), so one row's values are live at a time
      constexpr int NLD = EB == 4 ? 2 : 1;
      uint4 raw[4][NLD];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < NLD; ++c)
          raw[i][c] = reinterpret_cast<const uint4*>(xb + ((r0 + 4 * rg + i) * p.ld_x + cc) * EB)[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        AbsMax<DT> ami;
        float fr[8];
#pragma unroll
        for (int c = 0; c < NLD; ++c) ami.add(raw[i][c]);
        if constexpr (DT == kF32) {
          const uint4 lo = raw[i][0], hi = raw[i][NLD - 1];
          fr[0] = __uint_as_float(lo.x); fr[1] = __uint_as_float(lo.y); fr[2] = __uint_as_float(lo.z);
          fr[3] = __uint_as_float(lo.w); fr[4] = __uint_as_float(hi.x); fr[5] = __uint_as_float(hi.y);
          fr[6] = __uint_as_float(hi.z); fr[7] = __uint_as_float(hi.w);
        } else {
          const uint4 v = raw[i][0];
          widen2<DT>(v.x, fr[0], fr[1]); widen2<DT>(v.y, fr[2], fr[3]);
          widen2<DT>(v.z, fr[4], fr[5]); widen2<DT>(v.w, fr[6], fr[7]);
        }
        const bool rnan = ami.has_nan();
        const float rmax = rnan ? nan_free_absmax<8>(fr) : ami.value();
        amax = fmaxf(amax, rmax);
        const bool inrange = !rnan && sreg && rmax * fabsf(s) <= FmtTraits<FMT>::kMax;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float q0 = fr[4 * h] * s, q1 = fr[4 * h + 1] * s, q2 = fr[4 * h + 2] * s, q3 = fr[4 * h + 3] * s;
          if (inrange) rw[i][h] = cvt4_inrange<FMT>(q0, q1, q2, q3);
          else if (!rnan && sreg) rw[i][h] = cvt4<FMT>(q0, q1, q2, q3);
          else rw[i][h] = enc4_exact<FMT>(q0, q1, q2, q3);
        }
      }
    } else {
      AbsMax<DT> am;
      bool all_full = true;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + 4 * rg + i;
        const char* src = xb + (r * p.ld_x + cc) * EB;
        const bool full = AL || (r < p.rows && cc + 8 <= p.cols);  // vector loads, realigned if the row start is not
        all_full &= full;
        if (full) {
          if constexpr (DT == kF32) {
            uint4 ab[2];
            load16_any<2>(src, ab);
            const uint4 a = ab[0], b = ab[1];
            am.add(a);
            am.add(b);
            f[i][0] = __uint_as_float(a.x); f[i][1] = __uint_as_float(a.y);
            f[i][2] = __uint_as_float(a.z); f[i][3] = __uint_as_float(a.w);
            f[i][4] = __uint_as_float(b.x); f[i][5] = __uint_as_float(b.y);
            f[i][6] = __uint_as_float(b.z); f[i][7] = __uint_as_float(b.w);
          } else {
            uint4 a1[1];
            load16_any<1>(src, a1);
            const uint4 a = a1[0];
            am.add(a);
            widen2<DT>(a.x, f[i][0], f[i][1]); widen2<DT>(a.y, f[i][2], f[i][3]);
            widen2<DT>(a.z, f[i][4], f[i][5]); widen2<DT>(a.w, f[i][6], f[i][7]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            f[i][e] = (r < p.rows && cc + e < p.cols) ? load1<DT>(p.x, r * p.ld_x + cc + e) : 0.0f;
        }
      }
      bool nan;
      float camax;
      if (all_full) {  // every element came through a vector load
        nan = am.has_nan();
        camax = nan ? nan_free_absmax<32>(&f[0][0]) : am.value();
      } else {
        nan = false;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) nan |= f[i][e] != f[i][e];
        camax = nan_free_absmax<32>(&f[0][0]);
      }
      amax = fmaxf(amax, camax);
      if (early) {  // uniform over the workgroup
        const float bm = block_max<kTileThreads>(amax, red);
        if (t == 0) pub = ring_publish(p.ring, p.H, bm);
        pubd = true;
      }
      if (!nan && sreg && camax * fabsf(s) <= FmtTraits<FMT>::kMax) {
        // no clamp needed: fl32(|x| |s|) <= fl32(camax |s|) (monotonic rounding)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            rw[i][h] = cvt4_inrange<FMT>(f[i][4 * h] * s, f[i][4 * h + 1] * s, f[i][4 * h + 2] * s,
                                         f[i][4 * h + 3] * s);
      } else if (!nan && sreg) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            rw[i][h] = cvt4<FMT>(f[i][4 * h] * s, f[i][4 * h + 1] * s, f[i][4 * h + 2] * s, f[i][4 * h + 3] * s);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            rw[i][h] = enc4_exact<FMT>(f[i][4 * h] * s, f[i][4 * h + 1] * s, f[i][4 * h + 2] * s,
                                       f[i][4 * h + 3] * s);
      }
    }

    if (early && !pubd) {  // uniform over the workgroup
      const float bm = block_max<kTileThreads>(amax, red);
      if (t == 0) pub = ring_publish(p.ring, p.H, bm);
    }
    if constexpr (MODE == kRow || MODE == kDual) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + 4 * rg + i;
        if (!AL && r >= p.rows) continue;
        uint8_t* dst = p.out_row + r * p.ld_row + cc;
        if (AL || (cc + 8 <= p.cols && ((reinterpret_cast<uintptr_t>(dst) & 7u) == 0))) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(rw[i][0], rw[i][1]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (cc + e < p.cols) dst[e] = (uint8_t)(rw[i][e >> 2] >> (8 * (e & 3)));
        }
      }
    }

    if constexpr (MODE == kTrans || MODE == kDual) {
      // 4x8 bytes -> 8 column words (rows 4rg..4rg+3 of column 8cg+e)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t col[4];
        transpose4x4_bytes(rw[0][h], rw[1][h], rw[2][h], rw[3][h], col);
#pragma unroll
        for (int k = 0; k < 4; ++k) lds_t[lds_t_index(8 * cg + 4 * h + k, rg)] = col[k];
      }
      if constexpr (BG) {
        // bias gradient: fp64 column sums of the raw values -- this thread's 4
        // rows in order, parked in LDS by row group; after the barrier one
        // thread per column adds the 32 row groups in order
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          double v = (double)f[0][e];
#pragma unroll
          for (int i = 1; i < 4; ++i) v += (double)f[i][e];
          bg_part[bg_index(rg, 8 * cg + e)] = v;
        }
      }
      __syncthreads();
      if constexpr (BG) {
        if (t < kTileC && c0 + t < p.cols) {
          double v = bg_part[bg_index(0, t)];
#pragma unroll
          for (int g = 1; g < kTileR / 4; ++g) v += bg_part[bg_index(g, t)];
          p.bias_ws[(r0 / kTileR) * p.cols + c0 + t] = v;
        }
      }
      // 64 transposed rows (one per input column) x 128 bytes; lane: row cl, 16 bytes at 16q
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const int cl = (t >> 3) + 32 * pass, q = t & 7;
        const int64_t c = c0 + cl;
        const int64_t rr = r0 + 16 * q;
        if (AL || (c < p.cols && rr < p.rows)) {
          const uint4 v = *reinterpret_cast<const uint4*>(&lds_t[lds_t_index(cl, 4 * q)]);
          uint8_t* dst = p.out_t + c * p.ld_t + rr;
          if (AL || (rr + 16 <= p.rows && ((reinterpret_cast<uintptr_t>(dst) & 15u) == 0))) {
            *reinterpret_cast<uint4*>(dst) = v;
          } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if (rr + e < p.rows) dst[e] = (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
          }
        }
      }
      __syncthreads();  // LDS reused by the next tile
    }
  }
  if constexpr (MODE != kRow && !DYN) {
    if (early) {
      ring_block_finish<FMT>(p.ring, p.H, pub, s, p.scale_inv_out, p.amax_out, reinterpret_cast<uint32_t*>(red));
      return;
    }
  }
  quant_block_done<FMT, kTileThreads, DYN>(p, amax, s, red);
}

// Persistent form (quantize_tiled_pf).  One tile's raw input for this thread: rows 4rg..4rg+3 at columns
// 8cg..8cg+7, as 16-byte loads (two per row for f32; realigned when the row
// segment does not start on 16 bytes) where the 8 columns lie inside the
// tensor; other rows are read element by element while the tile is processed.
template <int DT> struct TileRaw {
  static constexpr int kLoads = In<DT>::kBytes == 4 ? 2 : 1;
  uint4 v[4][kLoads];
  uint32_t full;  // bit i: row i came through vector loads
};

template <int DT, int FMT, int MODE, bool BG, bool DYN>
__global__ void __launch_bounds__(kTileThreads) quantize_tiled_pf(QuantArgs p, int64_t tiles_c, int64_t ntiles,
                                                                int64_t tiles_per_block) {
  __shared__ float red[kTileThreads / 64];
  __shared__ __align__(16) uint32_t lds_t[(MODE == kRow) ? 1 : kTileC * 32];
  __shared__ double bg_part[BG ? kTileR / 4 * kTileC : 1];  // [row group][column], swizzled
  constexpr int EB = In<DT>::kBytes;
  constexpr int NLD = TileRaw<DT>::kLoads;
  const int t = threadIdx.x, cg = t & 7, rg = t >> 3;
  float amax = 0.0f;
  const char* xb = static_cast<const char*>(p.x);
  // Tiles are dealt round-robin (tile b, b + grid, b + 2 grid, ...): at any
  // time the workgroups work on one contiguous band of tiles, so the two
  // 64-column halves of a row's 128-byte code lines are written at about the
  // same time by neighbouring workgroups and leave the L2 as whole lines.
  // (Contiguous runs of tiles per workgroup wrote 15% more bytes for the dual
  // layout: the halves of a line split between runs were written far apart.)
  (void)tiles_per_block;
  const int64_t t_first = blockIdx.x, t_step = gridDim.x;

  auto load_tile = [&](int64_t tile, TileRaw<DT>& L) {
    int64_t r0, c0;
    tile_origin(tile, tiles_c, ntiles, r0, c0);
    const int64_t cc = c0 + 8 * cg;
    L.full = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = r0 + 4 * rg + i;
      const char* src = xb + (r * p.ld_x + cc) * EB;
      const bool full = r < p.rows && cc + 8 <= p.cols;
      L.full |= (uint32_t)full << i;
      if (full) load16_any<NLD>(src, L.v[i]);
    }
  };

  // In ring mode a workgroup publishes its amax at its last tile, once that
  // tile's values are in and before its codes are stored (see quantize_tiled).
  uint32_t pub = __builtin_nondeterministic_value(0u);  // read by thread 0 only
  auto process_tile = [&](int64_t tile, const TileRaw<DT>& L, float s, bool sreg) {
    int64_t r0, c0;
    tile_origin(tile, tiles_c, ntiles, r0, c0);
    const int64_t cc = c0 + 8 * cg;  // this thread's first column
    float f[4][8];
    AbsMax<DT> am;
    const bool all_full = L.full == 0xFu;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = r0 + 4 * rg + i;
      if ((L.full >> i) & 1u) {
        if constexpr (DT == kF32) {
          const uint4 a = L.v[i][0], b = L.v[i][NLD - 1];
          am.add(a);
          am.add(b);
          f[i][0] = __uint_as_float(a.x); f[i][1] = __uint_as_float(a.y);
          f[i][2] = __uint_as_float(a.z); f[i][3] = __uint_as_float(a.w);
          f[i][4] = __uint_as_float(b.x); f[i][5] = __uint_as_float(b.y);
          f[i][6] = __uint_as_float(b.z); f[i][7] = __uint_as_float(b.w);
        } else {
          const uint4 a = L.v[i][0];
          am.add(a);
          widen2<DT>(a.x, f[i][0], f[i][1]); widen2<DT>(a.y, f[i][2], f[i][3]);
          widen2<DT>(a.z, f[i][4], f[i][5]); widen2<DT>(a.w, f[i][6], f[i][7]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          f[i][e] = (r < p.rows && cc + e < p.cols) ? load1<DT>(p.x, r * p.ld_x + cc + e) : 0.0f;
      }
    }
    bool nan;
    float camax;
    if (all_full) {  // every element came through a vector load
      nan = am.has_nan();
      camax = nan ? nan_free_absmax<32>(&f[0][0]) : am.value();
    } else {
      nan = false;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) nan |= f[i][e] != f[i][e];
      camax = nan_free_absmax<32>(&f[0][0]);
    }
    amax = fmaxf(amax, camax);
    if constexpr (!DYN) {
      if (p.ring != nullptr && tile + t_step >= ntiles) {  // uniform over the workgroup
        const float bm = block_max<kTileThreads>(amax, red);
        if (t == 0) pub = ring_publish(p.ring, p.H, bm);
      }
    }
    uint32_t rw[4][2];  // row words: rw[i][h] = codes of row i, columns 4h..4h+3
    if (!nan && sreg && camax * fabsf(s) <= FmtTraits<FMT>::kMax) {
      // no clamp needed: fl32(|x| |s|) <= fl32(camax |s|) (monotonic rounding)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          rw[i][h] = cvt4_inrange<FMT>(f[i][4 * h] * s, f[i][4 * h + 1] * s, f[i][4 * h + 2] * s,
                                       f[i][4 * h + 3] * s);
    } else if (!nan && sreg) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          rw[i][h] = cvt4<FMT>(f[i][4 * h] * s, f[i][4 * h + 1] * s, f[i][4 * h + 2] * s, f[i][4 * h + 3] * s);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          rw[i][h] = enc4_exact<FMT>(f[i][4 * h] * s, f[i][4 * h + 1] * s, f[i][4 * h + 2] * s,
                                     f[i][4 * h + 3] * s);
    }

    if constexpr (MODE == kRow || MODE == kDual) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + 4 * rg + i;
        if (r >= p.rows) continue;
        uint8_t* dst = p.out_row + r * p.ld_row + cc;
        if (cc + 8 <= p.cols && ((reinterpret_cast<uintptr_t>(dst) & 7u) == 0)) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(rw[i][0], rw[i][1]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (cc + e < p.cols) dst[e] = (uint8_t)(rw[i][e >> 2] >> (8 * (e & 3)));
        }
      }
    }

    if constexpr (MODE == kTrans || MODE == kDual) {
      // 4x8 bytes -> 8 column words (rows 4rg..4rg+3 of column 8cg+e)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t col[4];
        transpose4x4_bytes(rw[0][h], rw[1][h], rw[2][h], rw[3][h], col);
#pragma unroll
        for (int k = 0; k < 4; ++k) lds_t[lds_t_index(8 * cg + 4 * h + k, rg)] = col[k];
      }
      if constexpr (BG) {
        // bias gradient: fp64 column sums of the raw values -- this thread's 4
        // rows in order, parked in LDS by row group; after the barrier one
        // thread per column adds the 32 row groups in order
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          double v = (double)f[0][e];
#pragma unroll
          for (int i = 1; i < 4; ++i) v += (double)f[i][e];
          bg_part[bg_index(rg, 8 * cg + e)] = v;
        }
      }
      __syncthreads();
      if constexpr (BG) {
        if (t < kTileC && c0 + t < p.cols) {
          double v = bg_part[bg_index(0, t)];
#pragma unroll
          for (int g = 1; g < kTileR / 4; ++g) v += bg_part[bg_index(g, t)];
          p.bias_ws[(r0 / kTileR) * p.cols + c0 + t] = v;
        }
      }
      // 64 transposed rows (one per input column) x 128 bytes; lane: row cl, 16 bytes at 16q
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const int cl = (t >> 3) + 32 * pass, q = t & 7;
        const int64_t c = c0 + cl;
        const int64_t rr = r0 + 16 * q;
        if (c < p.cols && rr < p.rows) {
          const uint4 v = *reinterpret_cast<const uint4*>(&lds_t[lds_t_index(cl, 4 * q)]);
          uint8_t* dst = p.out_t + c * p.ld_t + rr;
          if (rr + 16 <= p.rows && ((reinterpret_cast<uintptr_t>(dst) & 15u) == 0)) {
            *reinterpret_cast<uint4*>(dst) = v;
          } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if (rr + e < p.rows) dst[e] = (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
          }
        }
      }
      __syncthreads();  // LDS reused by the next tile
    }
  };

  // The tiles are software-pipelined: the loads of tile k + 1 are in flight
  // while tile k is encoded and stored (the copy at the end of an iteration
  // waits only for that prefetch).
  TileRaw<DT> cur, nxt;
  if (t_first < ntiles) load_tile(t_first, cur);
  const float s = read_scale<FMT, DYN>(p);  // after the first loads are out
  const bool sreg = scale_regular(s);
  for (int64_t tile = t_first; tile < ntiles; tile += t_step) {
    if (tile + t_step < ntiles) load_tile(tile + t_step, nxt);
    process_tile(tile, cur, s, sreg);
    cur = nxt;
  }
  if constexpr (!DYN) {
    if (p.ring != nullptr && t_first < ntiles) {
      ring_block_finish<FMT>(p.ring, p.H, pub, s, p.scale_inv_out, p.amax_out, reinterpret_cast<uint32_t*>(red));
      return;
    }
  }
  quant_block_done<FMT, kTileThreads, DYN>(p, amax, s, red);
}

// Fold alone / arming of a ring-less amax output.
template <int FMT> __global__ void amax_fold_kernel(uint32_t* ring, int H, const float* amax) {
  if (threadIdx.x < 64) ring_fold_wave<FMT>(ring, H, *amax, nullptr, 1.0f, nullptr);
}
__global__ void zero_word_kernel(float* p) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0.0f;
}

hipError_t launch_zero_word(float* p, hipStream_t st) {
  hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(64), 0, st, p);
  return hipGetLastError();
}

// ===========================================================================
// Current scaling, first pass.  Every workgroup writes the NaN-free max |x| of
// its share of the input to parts[blockIdx.x] as fp32 bits; the quantize pass
// that follows reads all partials in every wave (see read_scale), so there
// are no atomics and no workgroup ever waits on another.
// Contiguous input (ld_x == cols, or one row): the body of 16-byte chunks is
// shared grid-stride, kAmaxLoads chunks in flight per lane; the unaligned head
// and the ragged tail (fewer than 16 bytes each) go element by element in
// workgroup 0.  Strided rows: one wave per row at a time, same split per row.
// ===========================================================================
constexpr int kAmaxThreads = 256;
constexpr int kAmaxLoads = 8;
constexpr int kAmaxBlocksPerCU = 4;
constexpr int kDynSlots = 1024;  // partials capacity of the caller's workspace

// |x| of one element as a key that orders like the magnitude: the magnitude
// bits of the element's own format, NaN mapped to 0.
template <int DT> struct AmaxKey {
  static constexpr uint32_t kMag = DT == kF32 ? 0x7FFFFFFFu : 0x7FFFu;
  static constexpr uint32_t kInf = DT == kF32 ? 0x7F800000u : (DT == kF16 ? 0x7C00u : 0x7F80u);
  __device__ static __forceinline__ uint32_t key(uint32_t raw) {
    const uint32_t m = raw & kMag;
    return m > kInf ? 0u : m;
  }
  __device__ static __forceinline__ uint32_t chunk(const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (DT == kF32) {
        m = max(m, key(w[e]));
      } else {
        m = max(m, key(w[e]));  // low half (key masks the high half away)
        m = max(m, key(w[e] >> 16));
      }
    }
    return m;
  }
  __device__ static __forceinline__ uint32_t raw(const char* xb, int64_t i) {
    if constexpr (DT == kF32) return reinterpret_cast<const uint32_t*>(xb)[i];
    else return reinterpret_cast<const uint16_t*>(xb)[i];
  }
  // fp32 bits of the magnitude a key stands for (exact widening)
  __device__ static __forceinline__ uint32_t f32_bits(uint32_t k) {
    if constexpr (DT == kF32) return k;
    else if constexpr (DT == kBF16) return k << 16;
    else return __float_as_uint(f16_to_f32(k));
  }
};

// Key max of n contiguous elements at xb, spread over `nthr` threads of which
// this is number `tid`; 16-byte chunks in the middle, elements at the ends.
template <int DT>
__device__ __forceinline__ uint32_t segment_amax_key(const char* xb, int64_t n, int64_t tid, int64_t nthr) {
  using K = AmaxKey<DT>;
  constexpr int EB = In<DT>::kBytes, EPC = 16 / EB;
  const int64_t lead = (int64_t)(((16u - (reinterpret_cast<uintptr_t>(xb) & 15u)) & 15u) / EB);
  const int64_t head = lead < n ? lead : n;
  const int64_t nch = (n - head) / EPC;
  const int64_t tail0 = head + nch * EPC;
  const uint4* body = reinterpret_cast<const uint4*>(xb + head * EB);
  uint32_t m = 0;
  // batches of kAmaxLoads chunks per thread, all loads issued before any is
  // used; past the end a thread re-reads the last chunk (harmless for a max),
  // so the loads stay unconditional
  for (int64_t c = tid; c < nch; c += kAmaxLoads * nthr) {
    uint4 v[kAmaxLoads];
#pragma unroll
    for (int j = 0; j < kAmaxLoads; ++j) {
      const int64_t i = c + j * nthr;
      v[j] = body[i < nch ? i : nch - 1];
    }
#pragma unroll
    for (int j = 0; j < kAmaxLoads; ++j) m = max(m, K::chunk(v[j]));
  }
  if (tid < EPC) {
    if (tid < head) m = max(m, K::key(K::raw(xb, tid)));
    if (tail0 + tid < n) m = max(m, K::key(K::raw(xb, tail0 + tid)));
  }
  return m;
}

template <int DT>
__global__ void __launch_bounds__(kAmaxThreads) amax_partials(const void* x, int64_t rows, int64_t cols,
                                                             int64_t ld_x, uint32_t* parts) {
  using K = AmaxKey<DT>;
  constexpr int EB = In<DT>::kBytes;
  __shared__ uint32_t red[kAmaxThreads / 64];
  const char* xb = static_cast<const char*>(x);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t m = 0;
  if (ld_x == cols || rows == 1) {
    const int64_t nthr = (int64_t)gridDim.x * kAmaxThreads;
    const int64_t tid = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x;
    m = segment_amax_key<DT>(xb, rows * cols, tid, nthr);
  } else {
    const int64_t nw = (int64_t)gridDim.x * (kAmaxThreads / 64);
    for (int64_t r = (int64_t)blockIdx.x * (kAmaxThreads / 64) + wid; r < rows; r += nw)
      m = max(m, segment_amax_key<DT>(xb + r * ld_x * EB, cols, lane, 64));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if (lane == 0) red[wid] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = red[0];
#pragma unroll
    for (int w = 1; w < kAmaxThreads / 64; ++w) b = max(b, red[w]);
    parts[blockIdx.x] = K::f32_bits(b);
  }
}

// ===========================================================================
// Host launchers.
// ===========================================================================
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Grids (measured on MI355X, kernel trace, bf16 8192 x 1536 and 8192 x 6912):
// while every workgroup can take a single group / tile within
// kOneShotBlocksPerCU workgroups per CU, the one-shot kernels run (low
// registers, everything in flight at once); larger tensors go to persistent
// workgroups, kPersistBlocksPerCU per CU, each streaming a contiguous share
// with the next group / tile in flight.  FP8MI_Q_BPC overrides the
// persistent count for tuning.
constexpr int kOneShotBlocksPerCU = 8;
constexpr int kPersistBlocksPerCU = 3;
// An explicit scale with amax_out: every workgroup's atomic max lands on the
// caller's one word and these serialise (~12 ns each), so the row kernel
// then runs persistent with one workgroup per CU (bf16 8192 x 1536: 27 ->
// 12.3 us).  The tiled kernels keep their grids: persistent at one per CU
// they were as slow (transposed 19.4 us) or slower (dual 23.2 against 21.8).
constexpr int kAmaxOutBlocksPerCU = 1;

// Whole aligned tiles for the one-shot transposed / dual kernel (its AL form).
template <int DT> static bool tiles_aligned(const QuantArgs& p, int mode) {
  constexpr int EB = In<DT>::kBytes;
  const auto a = [](const void* q, unsigned m) { return (reinterpret_cast<uintptr_t>(q) & m) == 0; };
  if (p.rows % kTileR != 0 || p.cols % kTileC != 0) return false;
  if (!a(p.x, 15u) || ((p.ld_x * EB) & 15) != 0) return false;
  if (mode == kDual && (!a(p.out_row, 7u) || (p.ld_row & 7) != 0)) return false;
  return a(p.out_t, 15u) && (p.ld_t & 15) == 0;
}

template <int DT, int FMT, int M, bool BG, bool DYN>
static void launch_tiled(bool one_shot, dim3 grid, hipStream_t st, const QuantArgs& p, int64_t tiles_c,
                         int64_t ntiles, int64_t tpb) {
  if (one_shot) {
    // The AL form measured faster for transposed grids of every size, for
    // dual grids of up to 3 workgroups per CU (bf16 x 1536 columns, graph
    // replay: 4096 rows 10.2 -> 8.9 us) and for current-scaling dual passes
    // (8192 rows: the call 17.5 -> 16.9 us); slower for denser dual grids
    // with a ring or an explicit scale (6144 rows 11.5 -> 11.9, 8192 rows
    // 13.4 -> 14.6 us).
    const bool al_grid = M == kTrans || DYN || ntiles <= 3 * (int64_t)device_cu_count();
    if (M != kRow && al_grid && tiles_aligned<DT>(p, M))
      hipLaunchKernelGGL((quantize_tiled<DT, FMT, M, BG, DYN, true>), grid, dim3(kTileThreads), 0, st, p, tiles_c,
                         ntiles, tpb);
    else
      hipLaunchKernelGGL((quantize_tiled<DT, FMT, M, BG, DYN, false>), grid, dim3(kTileThreads), 0, st, p, tiles_c,
                         ntiles, tpb);
  } else {
    hipLaunchKernelGGL((quantize_tiled_pf<DT, FMT, M, BG, DYN>), grid, dim3(kTileThreads), 0, st, p, tiles_c, ntiles,
                       tpb);
  }
}

template <int DT, int FMT, bool DYN>
static hipError_t launch_dt_fmt(const QuantArgs& p, int mode, hipStream_t st) {
  const int ncu = device_cu_count();
  static const int persist_env = env_int_in("FP8MI_Q_BPC", 1, 16, kPersistBlocksPerCU);
  const bool word_amax = !DYN && !p.ring && p.amax_out;  // one caller word takes every block's maximum
  const int64_t n = p.rows * p.cols;
  const bool contiguous_row = mode == kRow && p.ld_x == p.cols && p.ld_row == p.cols &&
                              (reinterpret_cast<uintptr_t>(p.x) & 15u) == 0 &&
                              (reinterpret_cast<uintptr_t>(p.out_row) & 15u) == 0;
  if (contiguous_row || n == 0) {
    const int64_t steps = cdiv(n, kFlatBlockStep);
    const int persist_bpc = word_amax ? kAmaxOutBlocksPerCU : persist_env;
    if (!word_amax && steps <= (int64_t)ncu * kOneShotBlocksPerCU * kFlatUnroll) {
      const int64_t spb = kFlatUnroll, blocks = steps == 0 ? 1 : cdiv(steps, spb);
      hipLaunchKernelGGL((quantize_flat<DT, FMT, false, DYN>), dim3((unsigned)blocks), dim3(kFlatThreads), 0, st, p, n,
                         spb);
    } else {
      const int64_t spb = cdiv(steps, (int64_t)ncu * persist_bpc), blocks = cdiv(steps, spb);
      hipLaunchKernelGGL((quantize_flat<DT, FMT, true, DYN>), dim3((unsigned)blocks), dim3(kFlatThreads), 0, st, p, n,
                         spb);
    }
    return hipGetLastError();
  }
  const int64_t tiles_c = cdiv(p.cols, kTileC);
  const int64_t ntiles = cdiv(p.rows, kTileR) * tiles_c;
  const bool one_shot = ntiles <= (int64_t)ncu * kOneShotBlocksPerCU;
  const int64_t tpb = one_shot ? 1 : cdiv(ntiles, (int64_t)ncu * persist_env);
  // persistent: as many workgroups as before (ceil(ntiles / tpb)), tiles dealt round-robin
  const dim3 grid((unsigned)cdiv(ntiles, tpb));
  switch (mode) {
    case kRow: launch_tiled<DT, FMT, kRow, false, DYN>(one_shot, grid, st, p, tiles_c, ntiles, tpb); break;
    case kTrans: launch_tiled<DT, FMT, kTrans, false, DYN>(one_shot, grid, st, p, tiles_c, ntiles, tpb); break;
    default:
      if constexpr (DT != kF32 && !DYN) {
        if (p.bias_ws) {
          launch_tiled<DT, FMT, kDual, true, false>(one_shot, grid, st, p, tiles_c, ntiles, tpb);
          break;
        }
      }
      launch_tiled<DT, FMT, kDual, false, DYN>(one_shot, grid, st, p, tiles_c, ntiles, tpb);
      break;
  }
  return hipGetLastError();
}

template <int FMT, bool DYN> static hipError_t launch_fmt(const QuantArgs& p, int dt, int mode, hipStream_t st) {
  switch (dt) {
    case kF32: return launch_dt_fmt<kF32, FMT, DYN>(p, mode, st);
    case kF16: return launch_dt_fmt<kF16, FMT, DYN>(p, mode, st);
    default: return launch_dt_fmt<kBF16, FMT, DYN>(p, mode, st);
  }
}

hipError_t launch_quantize(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld_x, int fmt, int mode,
                           uint8_t* out_row, int64_t ld_row, uint8_t* out_t, int64_t ld_t, const float* scale,
                           uint32_t* ring, int H, float* scale_inv_out, float* amax_out, hipStream_t st,
                           double* bias_ws) {
  QuantArgs p{x, rows, cols, ld_x, out_row, ld_row, out_t, ld_t, scale, ring, H, scale_inv_out, amax_out, bias_ws,
              nullptr, 0};
  if (!ring && amax_out) {
    hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(64), 0, st, amax_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return fmt == kE4M3 ? launch_fmt<kE4M3, false>(p, dt, mode, st) : launch_fmt<kE5M2, false>(p, dt, mode, st);
}

// Current scaling: the partials pass, then the ordinary quantize kernels with
// the scale measured from the partials.
hipError_t launch_quantize_dynamic(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                                   int mode, uint8_t* out_row, int64_t ld_row, uint8_t* out_t, int64_t ld_t,
                                   float* scale_inv_out, float* amax_out, uint32_t* parts, hipStream_t st) {
  const int ncu = device_cu_count();
  static const int amax_bpc = env_int_in("FP8MI_AMAX_BPC", 1, 16, kAmaxBlocksPerCU);
  const int eb = dt == kF32 ? 4 : 2;
  // as few load batches per thread as the cap allows, spread evenly (a
  // half-filled last batch would cost a whole extra round trip)
  const int64_t chunks = rows * cols * eb / 16 + 1;
  const int64_t per_block = (int64_t)kAmaxThreads * kAmaxLoads;
  const int64_t cap = (int64_t)ncu * amax_bpc < kDynSlots ? (int64_t)ncu * amax_bpc : kDynSlots;
  const int64_t batches = cdiv(chunks, cap * per_block);
  int64_t nb = cdiv(chunks, per_block * batches);
  if (nb > cap) nb = cap;
  if (!(ld_x == cols || rows == 1)) {
    const int64_t rb = cdiv(rows, kAmaxThreads / 64);  // a wave per row: no more blocks than rows / 4
    if (nb > rb) nb = rb;
  }
  if (nb < 1) nb = 1;
  switch (dt) {
    case kF32: hipLaunchKernelGGL(amax_partials<kF32>, dim3((unsigned)nb), dim3(kAmaxThreads), 0, st, x, rows, cols,
                                  ld_x, parts); break;
    case kF16: hipLaunchKernelGGL(amax_partials<kF16>, dim3((unsigned)nb), dim3(kAmaxThreads), 0, st, x, rows, cols,
                                  ld_x, parts); break;
    default: hipLaunchKernelGGL(amax_partials<kBF16>, dim3((unsigned)nb), dim3(kAmaxThreads), 0, st, x, rows, cols,
                                ld_x, parts); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  QuantArgs p{x, rows, cols, ld_x, out_row, ld_row, out_t, ld_t, nullptr, nullptr, 0, scale_inv_out, amax_out,
              nullptr, parts, (int)nb};
  return fmt == kE4M3 ? launch_fmt<kE4M3, true>(p, dt, mode, st) : launch_fmt<kE5M2, true>(p, dt, mode, st);
}

hipError_t launch_amax_fold(uint32_t* ring, int H, const float* amax, int fmt, hipStream_t st) {
  if (fmt == kE4M3) hipLaunchKernelGGL(amax_fold_kernel<kE4M3>, dim3(1), dim3(64), 0, st, ring, H, amax);
  else hipLaunchKernelGGL(amax_fold_kernel<kE5M2>, dim3(1), dim3(64), 0, st, ring, H, amax);
  return hipGetLastError();
}

}  // namespace fp8mi
