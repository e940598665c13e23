// The per-tensor-scaled fp8 GEMM kernel template shared by the bf16-output
// (mm_fp8.hip), fp8-output (quantizing epilogue, mm_fp8_q8.hip) and K-major
// (layout tags, mm_fp8_km.hip) translation units, which alone include it.
#pragma once
#include "fp8mi_device.h"
#include "fp8mi_internal.h"

namespace fp8mi {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBK = 128;
constexpr int kMmThreads = 256;

// LDS tiles: rows of kBK = 128 bytes; the 16-byte chunk c of row r sits at
// chunk position c ^ swz(r).  gfx950 serves a ds_read_b128 16 lanes per cycle
// from 64 four-byte banks, each half-wave in two cycles split by the parity
// of lane bits 2..4 (measured with the LDS bank-conflict counter).  In an
// MFMA fragment read lane l reads row l%16, chunk 2(l/16) + h; swz(r) =
// ((r >> 1) & 1) | (r & 4) puts every such cycle's 16 reads on 16 distinct
// 16-byte bank groups (row parity picks the 128-byte half, the chunk
// position the group within it).
__device__ __forceinline__ int swz(int row) { return ((row >> 1) & 1) | (row & 4); }

// K-major operand tiles (an operand given as [K, rows], the tile's rows
// contiguous): LDS holds 128 k-rows of W bytes (CPR = W / 16 chunks each);
// the 16-byte chunk c of k-row kr sits at chunk position
// (c + rot(kr)) mod CPR, rot(kr) = (kr & 7) + 8 * bit 5 of kr -- a
// permutation for any CPR (192-byte rows included).  A fragment read (below)
// touches 8 consecutive k-rows per 16-lane group at one chunk: the rotation
// puts them on 8 distinct 4-bank groups for W = 128, 192 and 256, and bit 5
// (which separates the lane groups 0/2 from 1/3) moves the other half-wave
// onto the remaining banks.
template <int CPR> __device__ __forceinline__ int km_pos(int c, int kr) {
  return (c + (kr & 7) + (((kr >> 5) & 1) << 3)) % CPR;
}

typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i* lds_v2i_ptr;

// MFMA operand fragment (lane l: tile row rb + l%16, k = 32(l/16) .. +31)
// from a K-major tile with ds_read_b64_tr_b8.  Measured lane layout of that
// instruction: within each group of 16 lanes, output lane 8h + c receives in
// byte j the byte c of the 8 bytes addressed by lane 2j + h.  So lane a = 2j + h
// of a group addresses k-row kb + j at column rb + 8h, and every lane receives
// its own row's 8 consecutive k; four reads cover k = 32g .. 32g + 31.
template <int W> __device__ __forceinline__ v8i lds_frag_km(const uint8_t* S, int rb, int lane) {
  const int g = lane >> 4, a = lane & 15, j = a >> 1, h = a & 1;
  v8i r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int kr = 32 * g + 8 * q + j;
    const int pos = km_pos<W / 16>(rb >> 4, kr);
    const v2i d = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_ptr)(S + kr * W + pos * 16 + 8 * h));
    r[2 * q] = d[0];
    r[2 * q + 1] = d[1];
  }
  return r;
}

__device__ __forceinline__ v8i lds_frag(const uint8_t* S, int row, int g) {
  const int sw = swz(row);
  const uint4 lo = *reinterpret_cast<const uint4*>(S + row * kBK + (((2 * g) ^ sw) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(S + row * kBK + (((2 * g + 1) ^ sw) << 4));
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// Exact fp32 value of an fp8 code (OCP E4M3: 2^(e-7)(1 + m/8), subnormal
// m 2^-9, S.1111.111 NaN; E5M2: 2^(e-15)(1 + m/4), subnormal m 2^-16,
// exponent 31 inf / NaN), assembled from the fields.
template <int FMT> __device__ __forceinline__ float dec_fp8(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24;
  if constexpr (FMT == kE4M3) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    if (e == 15u && m == 7u) return __uint_as_float(sign | 0x7FC00000u);
    if (e == 0u) return __uint_as_float(sign | __float_as_uint((float)m * 0.001953125f));
    return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
  } else {
    const uint32_t e = (c >> 2) & 31u, m = c & 3u;
    if (e == 31u) return __uint_as_float(sign | (m ? 0x7FC00000u : 0x7F800000u));
    if (e == 0u) return __uint_as_float(sign | __float_as_uint((float)m * 1.52587890625e-05f));
    return __uint_as_float(sign | ((e + 112u) << 23) | (m << 21));
  }
}

// Bias element j as the epilogue adds it: a bf16 / fp16 / fp32 bias widened
// exactly, or an fp8-stored bias dequantized by one fp32 multiply with the
// bias scale (bscale = *p.bias_scale, read once per workgroup).  Split into
// the load of the stored bits and their decoding, so a kernel can issue the
// load long before it needs the value.
__device__ __forceinline__ uint32_t load_bias_bits(const MmArgs& p, int64_t j) {
  switch (p.bias_dtype) {
    case kF32: return static_cast<const uint32_t*>(p.bias)[j];
    case kBF16:
    case kF16: return static_cast<const uint16_t*>(p.bias)[j];
    default: return static_cast<const uint8_t*>(p.bias)[j];
  }
}
__device__ __forceinline__ float decode_bias(const MmArgs& p, uint32_t bits, float bscale) {
  switch (p.bias_dtype) {
    case kF32: return __uint_as_float(bits);
    case kBF16: return bf16_to_f32(bits);
    case kF16: return f16_to_f32(bits);
    case kFp8E4M3: return dec_fp8<kE4M3>(bits) * bscale;
    default: return dec_fp8<kE5M2>(bits) * bscale;
  }
}
__device__ __forceinline__ float load_bias(const MmArgs& p, int64_t j, float bscale) {
  return decode_bias(p, load_bias_bits(p, j), bscale);
}

template <int FA, int FB>
__device__ __forceinline__ v4f mfma_nt(const v8i& bfrag, const v8i& afrag, const v4f& c) {
  // first operand: B rows (format FB -> cbsz), second: A rows (format FA -> blgp).
  // Zero block-scale operands make the compiler emit the unscaled
  // v_mfma_f32_16x16x128_f8f6f4 (no scale prefix; 2-3% faster in an MFMA-bound
  // loop on MI355X, identical results).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfrag, afrag, c, FB, FA, 0, 0, 0, 0);
}

// Precise accumulation for short K.  The fp8 MFMA adds its 128 products in
// aligned groups of 8 k; inside a group every product is cut toward zero to
// a grid 2^-13 below the group's largest one, while the groups themselves
// and the accumulator are added to within one fp32 rounding (measured on
// MI355X with isolated products: one nonzero product per group gave errors
// below 2^-23.8 of the sum of the terms' magnitudes; two per group, up to
// 2^-13 of the largest term).  The precise form therefore issues eight MFMAs
// per fragment pair, MFMA s carrying byte q of the lane's fragment dword s at
// k position 8q of the lane's 32-k window and zeros elsewhere: one product
// per group, the same pairing of A and B bytes (both operands are spread
// alike), every k of the step covered once.  It costs 8x the MFMA work, so
// the dispatch uses it only while K is short, where the group truncation is
// a visible fraction of 1e-5 * sum |a b| and the GEMM is latency-bound.
constexpr int64_t kPreciseMaxK = 256;

__device__ __forceinline__ v8i spread_dword(const v8i& f, int s) {
  const uint32_t w = (uint32_t)f[s];
  v8i r;
  r[0] = (int)(w & 0xFFu); r[1] = 0;
  r[2] = (int)((w >> 8) & 0xFFu); r[3] = 0;
  r[4] = (int)((w >> 16) & 0xFFu); r[5] = 0;
  r[6] = (int)(w >> 24); r[7] = 0;
  return r;
}

template <int FA, int FB, bool PREC>
__device__ __forceinline__ v4f mma(const v8i& bfrag, const v8i& afrag, v4f c) {
  if constexpr (!PREC) {
    return mfma_nt<FA, FB>(bfrag, afrag, c);
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) c = mfma_nt<FA, FB>(spread_dword(bfrag, s), spread_dword(afrag, s), c);
    return c;
  }
}

// ===========================================================================
// LDS-DMA kernel template (mm_fp8_dma).  The 256 x 256 headline tile: 8 waves
// (2 along M x 4 along N), each wave 128 x 64 = 8 x 4 MFMA tiles (128 fp32
// accumulators per lane); K advances 128 bytes per step through two LDS
// stages (2 x 64 KiB).  The same template gives 256 x 192, 128 x 128 and,
// with three stages, 64 x 128 and 64 x 64.  The operands go from HBM/L2
// straight into LDS (buffer_load_dwordx4 ... lds): each load instruction
// fills 1 KiB = 8 tile rows, lane l writing 16 bytes at l * 16, so lane l
// fetches the 16-byte chunk that the XOR swizzle places there (row r0 + l/8,
// chunk (l%8) ^ swz(l/8)).  The loads of the next step(s) are in flight while
// this step's MFMAs run; one wait + barrier per step.  Rows past the matrix
// edge and chunks past K read as zero: their buffer offsets lie beyond the
// resource's byte count.
// Workgroups are renumbered so that the ones a single XCD runs (the hardware
// deals workgroup ids round-robin over the 8 XCDs) cover a compact block of
// tiles -- group_m tile rows by consecutive tile columns -- and share their
// A and B panels in that XCD's L2.
// ===========================================================================
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef int v4i __attribute__((ext_vector_type(4)));

// Raw buffer resource over `bytes` bytes from `base` (stride 0, dword3 as for
// all gfx9 raw buffers); reads at offsets >= bytes return zero.
__device__ __forceinline__ v4i buffer_rsrc(const void* base, int bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32) & 0xFFFF);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from a raw buffer straight into LDS at lds + 16 * lane.
// Written as asm so that the compiler's wait-count pass does not treat the
// LDS write as aliasing the current stage's ds_reads (it would otherwise wait
// for this prefetch before every read); the kernel waits for it explicitly
// (s_waitcnt vmcnt(0) + barrier) before the stage is read.  The asm has no
// register outputs; M0 is saved and restored around it.  The LDS address and
// the scalar offset are wave-uniform; readfirstlane keeps them in SGPRs.
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t lds, int voff, int soff) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff))
      : "memory");
}

// 32-bit arithmetic: the launch checks keep the tile count of a batch below
// 2^31, and 64-bit divisions cost a few hundred instructions per workgroup.
__device__ __forceinline__ void tile_coords(int64_t wg64, int64_t tiles_m64, int64_t tiles_n64, int group_m,
                                            int64_t& tm, int64_t& tn) {
  const uint32_t wg = (uint32_t)wg64, tiles_m = (uint32_t)tiles_m64, tiles_n = (uint32_t)tiles_n64;
  const uint32_t gm = (uint32_t)group_m;
  const uint32_t full = (tiles_m * tiles_n / 8u) * 8u;
  uint32_t id = wg;
  if (wg < full) id = (wg % 8u) * (full / 8u) + wg / 8u;  // same-XCD workgroups get consecutive ids
  const uint32_t per_group = gm * tiles_n;
  const uint32_t g = id / per_group, r = id % per_group;
  const uint32_t rows_here = (tiles_m - g * gm) < gm ? (tiles_m - g * gm) : gm;
  tm = (int64_t)(g * gm + r % rows_here);
  tn = (int64_t)(r / rows_here);
}

// Batched launches (grid x: the tiles of one batch, grid z: the batches):
// workgroups are dealt to the XCDs round-robin in launch order, so a batch's
// tiles would spread over several XCDs and each would fetch that batch's
// operands into its own L2.  The launch-order index is remapped so that the
// workgroups of one XCD take consecutive (batch, tile) pairs -- whole batches
// where a batch's tiles divide the XCD's share.  Returns the tile index within
// the batch in wg and the batch in bz.
__device__ __forceinline__ void batch_tile(int64_t& wg, int64_t& bz) {
  const uint64_t tiles = gridDim.x, total = tiles * gridDim.z;
  const uint64_t lin = (uint64_t)blockIdx.z * tiles + blockIdx.x;
  if (total <= 0xFFFFFFFFull) {  // 32-bit divisions (64-bit ones cost a few hundred instructions)
    const uint32_t t32 = (uint32_t)tiles, l32 = (uint32_t)lin, full = (uint32_t)total / 8u * 8u;
    const uint32_t id = l32 < full ? (l32 % 8u) * (full / 8u) + l32 / 8u : l32;
    bz = id / t32;
    wg = id % t32;
  } else {
    const uint64_t full = total / 8u * 8u;
    const uint64_t id = lin < full ? (lin % 8u) * (full / 8u) + lin / 8u : lin;
    bz = (int64_t)(id / tiles);
    wg = (int64_t)(id % tiles);
  }
}

// LAY: bit 0 -- A given K-major ([K, M], lda >= M), bit 1 -- B given K-major
// ([K, N], ldb >= N); otherwise the operand is [rows, K] (NT).
// Wait until at most r steps of LPW loads each are outstanding (r in [0, MAXR]).
template <int LPW, int MAXR> __device__ __forceinline__ void wait_steps(int r) {
  if constexpr (MAXR > 0) {
    if (r >= MAXR) {
      wait_vmem_n<LPW * MAXR>();
      return;
    }
    wait_steps<LPW, MAXR - 1>(r);
  } else {
    wait_vmem();
  }
}

// PREC: the precise accumulation above (short K).  DEEP > 0: that many LDS
// stages (DEEP - 1 steps of loads in flight) for the small tiles of
// problems that leave CUs idle, where each workgroup's chain of load
// latencies sets the time.
// LDS of one tile's workgroup, carved from one pool: the load stages (or
// the staged C tile, whichever is larger), the tile's bias, the reduction
// words of the quantizing epilogue.
template <int BM, int BN, int NWAVES, int DEEP> struct TileLds {
  static constexpr int kStages = DEEP > 0 ? DEEP : (BM * BN <= 64 * 128 ? 3 : 2);
  static constexpr int kStage = (BM + BN) * kBK;
  static constexpr int kCTile = BM * (BN + 8) * 2;
  static constexpr int kSmem = kStages * kStage > kCTile ? kStages * kStage : kCTile;
  static constexpr int kBias = kSmem;           // BN floats
  static constexpr int kRed = kBias + 4 * BN;   // NWAVES + 1 words
  static constexpr int kBytes = kRed + 4 * (NWAVES + 1);
};

// One BM x BN output tile at (m0, n0) of batch bz, with `pool` the
// workgroup's TileLds bytes.
template <int FA, int FB, int BM, int BN, int WAVES_M, int WAVES_N, int OUT, int LAY, bool PREC, int DEEP>
__device__ __forceinline__ void mm_tile(const MmArgs& p, const int64_t m0, const int64_t n0, const int64_t bz,
                                        uint8_t* pool) {
  constexpr bool KMA = (LAY & 1) != 0, KMB = (LAY & 2) != 0;
  constexpr int NWAVES = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TI = WM / 16, TJ = WN / 16;
  constexpr int STAGE = (BM + BN) * kBK;      // bytes per LDS stage
  // Loading waves: in the big tiles only waves 0 .. NWAVES / 2 - 1 (one per
  // SIMD) issue the LDS-DMA loads.  A wave stalls while its loads queue for
  // the CU's address unit (64 per K step); with the loads on one wave per
  // SIMD the other keeps the MFMA pipe fed meanwhile (alternating runs on one
  // box: 4096^3 56.0 -> 55.0 us, 8192^3 420 -> 403 us).
  constexpr int NLW = (BM * BN >= 256 * 192) ? NWAVES / 2 : NWAVES;
  constexpr int LA = BM / 8 / NLW;            // 1 KiB load instructions per loading wave for A
  constexpr int LB = BN / 8 / NLW;            // ... and for B
  static_assert(LA >= 1 && LB >= 1 && LA * 8 * NLW == BM && LB * 8 * NLW == BN, "tile / wave mismatch");
  static_assert(TI >= 1 && TJ >= 1, "wave tile below one MFMA tile");
  constexpr int CROW = BN + 8;                // bf16 per LDS row of the staged C tile (16 B pad)
  // LDS stages: two for the big tiles (2 x 64 KiB at 256 x 256); the small
  // 64 x 128 tile (24 KiB per stage, two workgroups per CU) keeps three, so
  // two K steps of loads are in flight -- small and skinny problems, which
  // leave CUs idle and are bound by load latency, gain most from it
  constexpr int STAGES = DEEP > 0 ? DEEP : (BM * BN <= 64 * 128 ? 3 : 2);
  static_assert(DEEP == 0 || (DEEP >= 3 && BM * BN <= 64 * 128), "deep pipelines are for the small tiles");
  constexpr int LPW = LA + LB;  // load instructions per wave and K step
  using Lds = TileLds<BM, BN, NWAVES, DEEP>;
  static_assert(Lds::kStages == STAGES && Lds::kStage == STAGE && Lds::kCTile == BM * CROW * 2, "LDS layout");
  uint8_t* const smem = pool;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / WAVES_N, wn = wid % WAVES_N;
  const int ext_a = (int)(KMA ? p.a_extent_km(m0) : p.a_extent_from(m0));
  const int ext_b = (int)(KMB ? p.b_extent_km(n0) : p.b_extent_from(n0));
  const v4i rsa = buffer_rsrc(p.a + bz * p.stride_a + (KMA ? m0 : m0 * p.lda), ext_a);
  const v4i rsb = buffer_rsrc(p.b + bz * p.stride_b + (KMB ? n0 : n0 * p.ldb), ext_b);
  // Lane l of a 1 KiB load fills LDS row r0 + l/8 (r0 a multiple of 8) at
  // chunk position l%8, so it fetches logical chunk (l%8) ^ swz(l/8).
  const int lr = lane >> 3, lc = (lane & 7) ^ swz(lr);
  // unsigned: offsets of rows past the edge may wrap; those rows' outputs are never stored
  const uint32_t lda = (uint32_t)p.lda, ldb = (uint32_t)p.ldb;
  const uint32_t va = lr * lda + 16 * lc, vb = lr * ldb + 16 * lc;
  const int K = (int)p.K;
  // K-major operands: load instruction ii fills LDS chunks 64 ii .. 64 ii + 63
  // of the stage; lane l's chunk q = 64 ii + l is position q % CPR of k-row
  // q / CPR, so it fetches the chunk c whose km_pos is that position.  The
  // step's k0 enters as the scalar offset k0 * ld.
  constexpr int CPR_A = BM / 16, CPR_B = BN / 16;

  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_ptr_t)smem;

  // The tile's bias: thread t < BN loads the stored bits of column n0 + t
  // now, so the load's latency passes under the K loop; the value is decoded
  // after the loop and shared through LDS.  (Loaded in the epilogue, the
  // latency showed once per tile, and once per element for 16- and 8-bit
  // biases: +4.5 µs (fp32) and +8.5 µs (bf16) at 8192 x 6912 x 1536.)
  static_assert(BN <= 64 * NWAVES, "one bias column per thread");
  float* const bias_s = reinterpret_cast<float*>(pool + Lds::kBias);
  const bool bias_col = p.bias != nullptr && tid < BN && n0 + tid < p.N;
  const uint32_t bias_bits = bias_col ? load_bias_bits(p, n0 + tid) : 0u;
  auto park_bias = [&]() {
    if (tid < BN) bias_s[tid] = bias_col ? decode_bias(p, bias_bits, p.bias_scale ? *p.bias_scale : 1.0f) : 0.0f;
  };

  // One stage of loads: a loading wave's LA instructions for A rows
  // (wid * LA + q) * 8 .. + 7 and LB for B rows (wid * LB + q) * 8 .. + 7.
  // The raw-buffer range check covers voffset + soffset (measured on MI355X):
  // a row past the matrix edge starts at or beyond the extent and a chunk at
  // or past K gets the extent itself as its voffset, so both read as zero.
  auto issue_all = [&](int stage, int k0) {
    if (wid >= NLW) return;
    const bool past = k0 + 16 * lc >= K;  // K tail: chunks at or past K read as zero
    const uint32_t as = smem_lds + stage * STAGE, bs = as + BM * kBK;
#pragma unroll
    for (int q = 0; q < (LA > LB ? LA : LB); ++q) {
      if (q < LA) {
        if constexpr (KMA) {
          const int qq = (wid * LA + q) * 64 + lane;
          const int kr = qq / CPR_A, pos = qq % CPR_A;  // k-row within the step; rows past K read zero
          const int rot = ((kr & 7) + (((kr >> 5) & 1) << 3)) % CPR_A;
          const uint32_t c = (uint32_t)((pos + CPR_A - rot) % CPR_A);  // inverse of km_pos
          dma16(rsa, as + (wid * LA + q) * 1024, k0 + kr >= K ? ext_a : (int)((uint32_t)kr * lda + 16 * c),
                (int)((uint32_t)k0 * lda));
        } else {
          const int r0 = (wid * LA + q) * 8;
          dma16(rsa, as + r0 * kBK, past ? ext_a : (int)(va + (uint32_t)r0 * lda), k0);
        }
      }
      if (q < LB) {
        if constexpr (KMB) {
          const int qq = (wid * LB + q) * 64 + lane;
          const int kr = qq / CPR_B, pos = qq % CPR_B;
          const int rot = ((kr & 7) + (((kr >> 5) & 1) << 3)) % CPR_B;
          const uint32_t c = (uint32_t)((pos + CPR_B - rot) % CPR_B);  // inverse of km_pos
          dma16(rsb, bs + (wid * LB + q) * 1024, k0 + kr >= K ? ext_b : (int)((uint32_t)kr * ldb + 16 * c),
                (int)((uint32_t)k0 * ldb));
        } else {
          const int r0 = (wid * LB + q) * 8;
          dma16(rsb, bs + r0 * kBK, past ? ext_b : (int)(vb + (uint32_t)r0 * ldb), k0);
        }
      }
    }
  };

  // Issue chunk c (of NCH) of one stage's loads: this wave's load
  // instructions c * LPW / NCH .. (c + 1) * LPW / NCH - 1 (A's LA first,
  // then B's LB).
  constexpr int NCH = 4;
  auto issue_chunk = [&](int stage, int k0, int c) {
    if (wid >= NLW) return;
    const bool past = k0 + 16 * lc >= K;
    const uint32_t as = smem_lds + stage * STAGE, bs = as + BM * kBK;
#pragma unroll
    for (int q = c * LPW / NCH; q < (c + 1) * LPW / NCH; ++q) {
      if (q < LA) {
        if constexpr (KMA) {
          const int qq = (wid * LA + q) * 64 + lane;
          const int kr = qq / CPR_A, pos = qq % CPR_A;
          const int rot = ((kr & 7) + (((kr >> 5) & 1) << 3)) % CPR_A;
          const uint32_t c2 = (uint32_t)((pos + CPR_A - rot) % CPR_A);
          dma16(rsa, as + (wid * LA + q) * 1024, k0 + kr >= K ? ext_a : (int)((uint32_t)kr * lda + 16 * c2),
                (int)((uint32_t)k0 * lda));
        } else {
          const int r0 = (wid * LA + q) * 8;
          dma16(rsa, as + r0 * kBK, past ? ext_a : (int)(va + (uint32_t)r0 * lda), k0);
        }
      } else {
        const int qb = q - LA;
        if constexpr (KMB) {
          const int qq = (wid * LB + qb) * 64 + lane;
          const int kr = qq / CPR_B, pos = qq % CPR_B;
          const int rot = ((kr & 7) + (((kr >> 5) & 1) << 3)) % CPR_B;
          const uint32_t c2 = (uint32_t)((pos + CPR_B - rot) % CPR_B);
          dma16(rsb, bs + (wid * LB + qb) * 1024, k0 + kr >= K ? ext_b : (int)((uint32_t)kr * ldb + 16 * c2),
                (int)((uint32_t)k0 * ldb));
        } else {
          const int r0 = (wid * LB + qb) * 8;
          dma16(rsb, bs + r0 * kBK, past ? ext_b : (int)(vb + (uint32_t)r0 * ldb), k0);
        }
      }
    }
  };

  v4f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int nk = (K + kBK - 1) / kBK;
  const int r16 = lane & 15, g = lane >> 4;
  auto frag_a = [&](const uint8_t* As, int i) -> v8i {
    return KMA ? lds_frag_km<BM>(As, wm * WM + 16 * i, lane) : lds_frag(As, wm * WM + 16 * i + r16, g);
  };
  auto frag_b = [&](const uint8_t* Bs, int j) -> v8i {
    return KMB ? lds_frag_km<BN>(Bs, wn * WN + 16 * j, lane) : lds_frag(Bs, wn * WN + 16 * j + r16, g);
  };
  if constexpr (STAGES == 2) {
    // Two stages, A fragments read two rows ahead.  Iteration kt enters with
    // step kt's B fragments and A fragments 0 and 1 in registers (A rows
    // rotate through four registers, ar[i % 4]) and half of step kt + 1's
    // loads issued; the other half goes out after rows 0 and 1.  After row
    // TI - 3 the wave waits for its reads of stage kt (the last A fragment
    // was read two rows earlier) and its loads of step kt + 1, and passes the
    // barrier: every wave is done with stage kt and step kt + 1 is visible.
    // Rows TI - 2 and TI - 1 run after the barrier while step kt + 1's first
    // two A fragments (into the registers rows TI - 4 and TI - 3 freed) and,
    // as each MFMA of the last row issues, its B fragments are read; then the
    // first half of step kt + 2's loads goes into stage kt, now free.  At the
    // last step these reads fetch the idle stage and go unused.
    static_assert(TI >= 4 && TI % 4 == 0, "two-stage schedule needs a multiple of four A rows per wave");
    v8i bf[TJ], ar[4];
    if (nk > 0) issue_all(0, 0);
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int j = 0; j < TJ; ++j) bf[j] = frag_b(smem + BM * kBK, j);
    ar[0] = frag_a(smem, 0);
    ar[1] = frag_a(smem, 1);
    // Where the second half of a step's loads goes (p.early_loads, chosen by
    // the launch): after rows 0 and 1 of the step before it (one round of
    // tiles, all workgroups in step), or right after the barrier's rows TI - 2
    // and TI - 1, a step earlier (several rounds).  Alternating runs on one
    // box: 4096^3 53.4 vs 54.5-55.4 us, while 8192^3 399 -> 387.5 us and
    // 8192 x 6912 x 1536 85.6 -> 83.6 us with the early form.
    const bool early = p.early_loads != 0;
    if (nk > 1) {
      issue_chunk(1, kBK, 0);
      issue_chunk(1, kBK, 1);
      if (early) {
        issue_chunk(1, kBK, 2);
        issue_chunk(1, kBK, 3);
      }
    }
    for (int kt = 0; kt < nk; ++kt) {
      const uint8_t* As = smem + (kt & 1) * STAGE;
      const uint8_t* An = smem + ((kt + 1) & 1) * STAGE;
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        if (i + 2 < TI) ar[(i + 2) & 3] = frag_a(As, i + 2);
        if (i == TI - 2) {  // after the barrier: step kt + 1's first two A fragments
          ar[(i + 2) & 3] = frag_a(An, 0);
          ar[(i + 3) & 3] = frag_a(An, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          acc[i][j] = mma<FA, FB, PREC>(bf[j], ar[i & 3], acc[i][j]);
          if (i == TI - 1) {
            __builtin_amdgcn_sched_barrier(0);
            bf[j] = frag_b(An + BM * kBK, j);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (!early && i < 2 && kt + 1 < nk) issue_chunk((kt + 1) & 1, (kt + 1) * kBK, 2 + i);
        if (early && i >= TI - 2 && kt + 2 < nk) issue_chunk(kt & 1, (kt + 2) * kBK, 2 + i - (TI - 2));
        if (i == TI - 3) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          wait_vmem();
          __syncthreads();
          if (kt + 2 < nk) {
            issue_chunk(kt & 1, (kt + 2) * kBK, 0);
            issue_chunk(kt & 1, (kt + 2) * kBK, 1);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // every wave passed the last barrier after its last read of a stage the
    // epilogue overwrites: wait for the idle-stage reads of the last step too
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    park_bias();
    __syncthreads();
  } else {
  // prologue: steps 0 .. STAGES-2 in flight; wait for step 0 only
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue_all(s, s * kBK);
  // step 0 must have landed; steps 1 .. min(STAGES - 2, nk - 1) may stay in flight
  wait_steps<LPW, STAGES - 2>(nk - 1 < STAGES - 2 ? nk - 1 : STAGES - 2);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const uint8_t* As = smem + (kt % STAGES) * STAGE;
    const uint8_t* Bs = As + BM * kBK;
    // the stage refilled here was last read in step kt - 1 (all waves passed
    // the barrier that ended it)
    if (kt + STAGES - 1 < nk) issue_all((kt + STAGES - 1) % STAGES, (kt + STAGES - 1) * kBK);
    v8i bfr[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j)
      bfr[j] = KMB ? lds_frag_km<BN>(Bs, wn * WN + 16 * j, lane) : lds_frag(Bs, wn * WN + 16 * j + r16, g);
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const v8i af = KMA ? lds_frag_km<BM>(As, wm * WM + 16 * i, lane) : lds_frag(As, wm * WM + 16 * i + r16, g);
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = mma<FA, FB, PREC>(bfr[j], af, acc[i][j]);
    }
    // step kt + 1 must have landed; the loads of steps kt + 2 .. (those
    // issued) may stay in flight
    {
      const int r = nk - 2 - kt;
      wait_steps<LPW, STAGES - 2>(r < 0 ? 0 : (r < STAGES - 2 ? r : STAGES - 2));
    }
    __syncthreads();
  }
  park_bias();
  __syncthreads();
  }

  // Epilogue: y = acc * fl32(sa * sb) + bias[j] in fp32, then one bf16
  // rounding (OUT < 0) or the output quantization (OUT = E4M3 / E5M2).
  const float sa = p.a_scale_inv ? *p.a_scale_inv : 1.0f;
  const float sb = p.b_scale_inv ? *p.b_scale_inv : 1.0f;
  const float sab = sa * sb;
  const int ng = lane >> 4;
  float bias_v[TJ][4];
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const float4 b4 = *reinterpret_cast<const float4*>(&bias_s[wn * WN + 16 * j + 4 * ng]);
    bias_v[j][0] = b4.x; bias_v[j][1] = b4.y; bias_v[j][2] = b4.z; bias_v[j][3] = b4.w;
  }
  if constexpr (OUT >= 0) {
    // Quantizing epilogue.  The output scale comes from the ring (read before
    // this workgroup's amax is published, so before the fold can replace it)
    // or from the caller.
    float* const red_c = reinterpret_cast<float*>(pool + Lds::kRed);
    uint8_t* C = static_cast<uint8_t*>(p.c) + bz * p.stride_c;
    const float s_c = p.c_ring ? __uint_as_float(p.c_ring[p.c_H]) : *p.c_scale;
    const bool sreg = scale_regular(s_c);
    const int rows_in = p.M - m0 < BM ? (int)(p.M - m0) : BM;  // rows / columns of the tile inside C
    const int cols_in = p.N - n0 < BN ? (int)(p.N - n0) : BN;
    const bool interior = rows_in == BM && cols_in == BN;
    // y = acc * fl32(sa * sb) + bias in fp32, in place, and the largest |y|
    // over the outputs inside C with NaN propagated (v_maximum3): a NaN
    // result says some output there is NaN
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(acc[i][j][r], sab, bias_v[j][r]);
    auto tile_max = [&](auto maxop) {
      float m = 0.0f;
      if (interior) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) m = maxop(m, fabsf(acc[i][j][r]));
      } else {
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const bool row_in = wm * WM + 16 * i + r16 < rows_in;
#pragma unroll
          for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (row_in && wn * WN + 16 * j + 4 * ng + r < cols_in) m = maxop(m, fabsf(acc[i][j][r]));
        }
      }
      return m;
    };
    float amax = tile_max([](float a, float b) { return __builtin_elementwise_maximum(a, b); });
    // Codes go to a [BM][BN + 16] byte tile in LDS (the stages are free after
    // the K loop), then whole rows leave in 16-byte pieces.  The encoder is
    // chosen once for the whole wave: the hardware conversion, or the integer
    // encoder when any lane holds a NaN output (the conversion's NaN code
    // differs) or the scale is not regular (y * s may be NaN where y is not).
    constexpr int CROW8 = BN + 16;
    uint8_t* Cs = smem;
    const bool fast = !__any(amax != amax) && sreg;
    // the amax leaves NaN out (fmaxf returns the other operand for a NaN)
    if (!fast) amax = tile_max([](float a, float b) { return fmaxf(a, b); });
    // With an output ring the workgroup's amax is published before any code is
    // encoded or stored (its atomic's round trip overlaps them); the tickets
    // follow the stores.
    uint32_t pub = __builtin_nondeterministic_value(0u);  // read by thread 0 only
    if (p.c_ring) {
      const float bmax = block_max<64 * NWAVES>(amax, red_c);
      if (threadIdx.x == 0) pub = ring_publish(p.c_ring, p.c_H, bmax);
    }
    // With no lane's fl32(amax |s|) above fmt_max no code needs the clamp:
    // fl32(|y| |s|) <= fl32(amax |s|) since rounding is monotonic.
    if (fast && !__any(amax * fabsf(s_c) > FmtTraits<OUT>::kMax)) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const v4f y = acc[i][j];
          *reinterpret_cast<uint32_t*>(Cs + (wm * WM + 16 * i + r16) * CROW8 + wn * WN + 16 * j + 4 * ng) =
              cvt4_inrange<OUT>(y[0] * s_c, y[1] * s_c, y[2] * s_c, y[3] * s_c);
        }
    } else if (fast) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const v4f y = acc[i][j];
          *reinterpret_cast<uint32_t*>(Cs + (wm * WM + 16 * i + r16) * CROW8 + wn * WN + 16 * j + 4 * ng) =
              cvt4<OUT>(y[0] * s_c, y[1] * s_c, y[2] * s_c, y[3] * s_c);
        }
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const v4f y = acc[i][j];
          *reinterpret_cast<uint32_t*>(Cs + (wm * WM + 16 * i + r16) * CROW8 + wn * WN + 16 * j + 4 * ng) =
              enc4_exact<OUT>(y[0] * s_c, y[1] * s_c, y[2] * s_c, y[3] * s_c);
        }
    }
    __syncthreads();
    {
      constexpr int LPR = BN / 16, RPW = 64 / LPR;
      const int sub = lane / LPR, cl = lane % LPR;
      const bool vec = (p.ldc % 16) == 0 && (reinterpret_cast<uintptr_t>(C) & 15u) == 0;
      if (interior && vec) {
#pragma unroll 4
        for (int rr = wid * RPW + sub; sub < RPW && rr < BM; rr += RPW * NWAVES) {
          const uint4 v = *reinterpret_cast<const uint4*>(Cs + rr * CROW8 + 16 * cl);
          *reinterpret_cast<uint4*>(C + (m0 + rr) * p.ldc + n0 + 16 * cl) = v;
        }
      } else {
        for (int rr = wid * RPW + sub; sub < RPW && rr < rows_in; rr += RPW * NWAVES) {
          const uint8_t* src = Cs + rr * CROW8 + 16 * cl;
          uint8_t* dst = C + (m0 + rr) * p.ldc + n0 + 16 * cl;
          if (vec && 16 * cl + 16 <= cols_in) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
          } else {
            for (int b = 0; b < 16 && 16 * cl + b < cols_in; ++b) dst[b] = src[b];
          }
        }
      }
    }
    // the cross-workgroup publication: the ring protocol's tickets (the last
    // workgroup folds), or an atomic max of this workgroup's amax into the
    // caller's word (zeroed before the launch)
    if (p.c_ring) {
      ring_block_finish<OUT>(p.c_ring, p.c_H, pub, s_c, p.c_scale_inv_out, p.c_amax_out,
                             reinterpret_cast<uint32_t*>(red_c + NWAVES));
    } else {
      const float bmax = block_max<64 * NWAVES>(amax, red_c);
      if (threadIdx.x == 0) {
        if (p.c_amax_out) publish_max(reinterpret_cast<uint32_t*>(p.c_amax_out), bmax);
        if (p.c_scale_inv_out && blockIdx.x == 0 && blockIdx.z == 0) *p.c_scale_inv_out = 1.0f / s_c;
      }
    }
    return;
  }
  uint16_t* C = static_cast<uint16_t*>(p.c) + bz * p.stride_c;
  // Interior tiles go out through LDS (the stages are free after the K loop):
  // each lane parks its 4-column pieces in a [256][256 + 8] bf16 tile, then
  // every wave stores whole 512-byte rows with 16-byte lanes.
  const bool interior = m0 + BM <= p.M && n0 + BN <= p.N && (p.ldc % 8) == 0 &&
                        ((reinterpret_cast<uintptr_t>(C) & 15u) == 0);
  if (interior) {
    uint16_t* Cs = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int lm = wm * WM + 16 * i + r16;
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        *reinterpret_cast<uint2*>(Cs + lm * CROW + wn * WN + 16 * j + 4 * ng) =
            bf16x4_rne(fmaf(acc[i][j][0], sab, bias_v[j][0]), fmaf(acc[i][j][1], sab, bias_v[j][1]),
                       fmaf(acc[i][j][2], sab, bias_v[j][2]), fmaf(acc[i][j][3], sab, bias_v[j][3]));
      }
    }
    __syncthreads();
    // BN / 8 lanes x 16 bytes per row; a wave stores RPW rows per step (lanes
    // past RPW * LPR idle when BN / 8 does not divide 64, e.g. BN = 192)
    constexpr int LPR = BN / 8, RPW = 64 / LPR;
    const int sub = lane / LPR, cl = lane % LPR;
    // fully unrolled: every LDS row read is in flight before the first store
    // (by four: 1-2.6% slower on 4096^3 and the linear's GEMMs)
#pragma unroll
    for (int rr = wid * RPW + sub; sub < RPW && rr < BM; rr += RPW * NWAVES) {
      const uint4 v = *reinterpret_cast<const uint4*>(Cs + rr * CROW + 8 * cl);
      *reinterpret_cast<uint4*>(C + (m0 + rr) * p.ldc + n0 + 8 * cl) = v;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int64_t gm = m0 + wm * WM + 16 * i + r16;
    if (gm >= p.M) continue;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t gn = n0 + wn * WN + 16 * j + 4 * ng;
      if (gn >= p.N) continue;
      const uint2 w = bf16x4_rne(fmaf(acc[i][j][0], sab, bias_v[j][0]), fmaf(acc[i][j][1], sab, bias_v[j][1]),
                                 fmaf(acc[i][j][2], sab, bias_v[j][2]), fmaf(acc[i][j][3], sab, bias_v[j][3]));
      uint16_t* dst = C + gm * p.ldc + gn;
      if (gn + 4 <= p.N && ((reinterpret_cast<uintptr_t>(dst) & 7u) == 0)) {
        *reinterpret_cast<uint2*>(dst) = w;
      } else {
        const uint32_t h[4] = {w.x & 0xFFFFu, w.x >> 16, w.y & 0xFFFFu, w.y >> 16};
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (gn + r < p.N) dst[r] = (uint16_t)h[r];
      }
    }
  }
}

template <int FA, int FB, int BM, int BN, int WAVES_M, int WAVES_N, int MIN_BLOCKS, int OUT, int LAY, bool PREC,
          int DEEP = 0>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, MIN_BLOCKS) mm_fp8_dma(MmArgs p, int64_t tiles_m,
                                                                                 int64_t tiles_n, int group_m) {
  __shared__ __align__(16) uint8_t pool[TileLds<BM, BN, WAVES_M * WAVES_N, DEEP>::kBytes];
  int64_t tm, tn, bz = 0, wg = blockIdx.x;
  if (gridDim.z > 1) batch_tile(wg, bz);
  tile_coords(wg, tiles_m, tiles_n, group_m, tm, tn);
  mm_tile<FA, FB, BM, BN, WAVES_M, WAVES_N, OUT, LAY, PREC, DEEP>(p, tm * BM, tn * BN, bz, pool);
}

// Mixed grid for a last round of 256 x 256 tiles that would leave most CUs
// idle: workgroups 0 .. tiles_m * tiles_n - 1 take the 256 x 256 tiles of
// columns [0, n_band), dispatched first; the rest take 128 x 256 tiles of
// the band [n_band, N), which start as CUs come free and take about half a
// big tile's time.  Both shapes sum every output's K in the same MFMA
// order, so the result equals the all-256 x 256 launch bit for bit.
template <int FA, int FB, int OUT, int LAY>
__global__ void __launch_bounds__(512, 1) mm_fp8_mixed(MmArgs p, int64_t tiles_m, int64_t tiles_n,
                                                       int64_t band_tiles_m, int64_t band_tiles_n, int64_t n_band,
                                                       int group_m) {
  using Big = TileLds<256, 256, 8, 0>;
  using Band = TileLds<128, 256, 8, 0>;
  __shared__ __align__(16) uint8_t pool[Big::kBytes > Band::kBytes ? Big::kBytes : Band::kBytes];
  const int64_t nbig = tiles_m * tiles_n;
  int64_t tm, tn;
  if ((int64_t)blockIdx.x < nbig) {
    tile_coords(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    mm_tile<FA, FB, 256, 256, 2, 4, OUT, LAY, false, 0>(p, tm * 256, tn * 256, 0, pool);
  } else {
    // nbig is a multiple of 8, so the band's own index keeps the XCD of blockIdx.x
    tile_coords((int64_t)blockIdx.x - nbig, band_tiles_m, band_tiles_n, group_m, tm, tn);
    mm_tile<FA, FB, 128, 256, 2, 4, OUT, LAY, false, 0>(p, tm * 128, n_band + tn * 256, 0, pool);
  }
}


// Tile dispatch (measured on MI355X over the shapes of the test configs):
// the 8-wave big-tile kernels whenever their tiles (x batch) cover at least
// 60% of the CUs -- one round of big tiles beats several rounds of small ones
// even with part of the chip idle -- choosing 256 x 192 over 256 x 256 when it
// needs less time per CU (the backward GEMMs of the 1536-wide linear get 256
// and 216 workgroups instead of 192 and 162, 10-11% faster), and the 64x128 /
// 4-wave kernel (two per CU, three LDS stages) below 60% -- or 64x64 when the
// 64x128 tiles number at most one per CU, and 64x32 (deep pipeline) when
// even the 64x64 tiles would fill at most half the CUs and K is long.
// 128x128 is reachable through FP8MI_MM_TILE=1 for tuning.  The first 128x128
// kernel remains for operands whose byte extent does not fit a 32-bit buffer
// offset.
template <int FA, int FB, int BM, int BN, int WM_, int WN_, int MINB, int OUT, int LAY = 0, bool PREC = false,
          int DEEP = 0>
static hipError_t launch_dma(const MmArgs& p0, hipStream_t st) {
  const int64_t tiles_m = (p0.M + BM - 1) / BM, tiles_n = (p0.N + BN - 1) / BN;
  const dim3 grid((unsigned)(tiles_m * tiles_n), 1, (unsigned)p0.batch);
  MmArgs p = p0;
  p.early_loads = tiles_m * tiles_n * p0.batch > (int64_t)device_cu_count();  // more than one round
  hipLaunchKernelGGL((mm_fp8_dma<FA, FB, BM, BN, WM_, WN_, MINB, OUT, LAY, PREC, DEEP>), grid, dim3(64 * WM_ * WN_),
                     0, st, p, tiles_m, tiles_n, 4);
  return hipGetLastError();
}

// FP8MI_MM_TILE: a forced tile for tuning (-1 when unset or invalid).
static inline int mm_forced_tile() {
  static const int forced = env_int_in("FP8MI_MM_TILE", 0, 8, -1);
  return forced == 4 ? -1 : forced;
}

// Columns of 256 x 256 tiles handed to the 128 x 256 band of mm_fp8_mixed,
// or 0 when the mixed grid does not apply: one batch, at least two rounds
// of 256 x 256 tiles with the last at most half full, the band the last
// ceil(last / tiles_m) tile columns, the big tiles left a multiple of 8 and
// the band's 128 x 256 tiles at most one per CU.  (8192 x 6912 x 1536: 864
// tiles on 256 CUs = 3 rounds + 96 -> 768 big tiles + a 8192 x 768 band of
// 192 tiles.)
static inline int64_t mixed_band_cols(const MmArgs& p, int ncu) {
  if (p.batch != 1) return 0;
  const int64_t tm = (p.M + 255) / 256, tn = (p.N + 255) / 256, t = tm * tn;
  const int64_t rounds = (t + ncu - 1) / ncu;
  if (rounds < 2) return 0;
  const int64_t last = t - (rounds - 1) * ncu;
  if (2 * last > ncu) return 0;
  const int64_t cb = (last + tm - 1) / tm;
  if (cb >= tn || (tm * (tn - cb)) % 8 != 0) return 0;
  return ((p.M + 127) / 128) * cb <= ncu ? cb : 0;
}

template <int FA, int FB, int OUT, int LAY> static hipError_t launch_mixed(const MmArgs& p0, int64_t cb,
                                                                            hipStream_t st) {
  MmArgs p = p0;
  p.early_loads = 1;  // at least two rounds
  const int64_t tiles_m = (p.M + 255) / 256, tiles_n = (p.N + 255) / 256 - cb;
  const int64_t band_m = (p.M + 127) / 128;
  const dim3 grid((unsigned)(tiles_m * tiles_n + band_m * cb), 1, 1);
  hipLaunchKernelGGL((mm_fp8_mixed<FA, FB, OUT, LAY>), grid, dim3(512), 0, st, p, tiles_m, tiles_n, band_m, cb,
                     tiles_n * 256, 4);
  return hipGetLastError();
}

static inline int pick_tile(const MmArgs& p, int ncu) {
  const int forced = mm_forced_tile();
  if (forced >= 0) return forced;
  const int64_t tm = (p.M + 255) / 256;
  const int64_t t256 = tm * ((p.N + 255) / 256) * p.batch, t192 = tm * ((p.N + 191) / 192) * p.batch;
  if (10 * (t256 > t192 ? t256 : t192) < 6 * (int64_t)ncu) {
    // small problems: 64 x 128 tiles, or 64 x 64 when even those would not
    // give every CU one (skinny shapes; measured 3-10% faster there, slower
    // once the 64 x 128 tiles fill the chip); with at most one 64 x 64 tile
    // per CU and a long K, its deep-pipeline form (8 stages, one workgroup
    // per CU: 64x8192x2048 8.13 -> 7.97 us, 128x4096x4096 12.5 -> 11.7 us; a
    // 6-stage 64 x 128 form was slower on every sweep shape)
    const int64_t t128 = ((p.M + 63) / 64) * ((p.N + 127) / 128) * p.batch;
    const int64_t t64 = ((p.M + 63) / 64) * ((p.N + 63) / 64) * p.batch;
    const bool long_k = p.K >= 6 * kBK;
    // with even the 64 x 64 tiles at most half a workgroup per CU and a long
    // K, 64 x 32 tiles (deep pipeline): twice the workgroups, each streaming
    // half the B panel (best of three runs, one box: 64x8192x2048 8.1 -> 7.5
    // us, 128x4096x4096 12.1 -> 10.3 us, 64x1536x6912 17.6 -> 14.5 us)
    if (long_k && 2 * t64 <= (int64_t)ncu) return 8;
    if (t128 <= (int64_t)ncu) return long_k && t64 <= (int64_t)ncu ? 6 : 5;
    return 2;
  }
  // per-CU time of the big-tile family: rounds of workgroups x the time of
  // one round, a 256 x 192 round taking ~0.9 of a 256 x 256 one (measured
  // per K step on MI355X; its MFMA work is 0.75 of it).  So 256 x 192 wins
  // when it needs no more rounds (the backward GEMMs of the 1536-wide
  // linear), 256 x 256 when it saves a round (8192 x 6912 x 1536: 4 rounds
  // instead of 5, 3% faster).
  const int64_t cost256 = ((t256 + ncu - 1) / ncu) * 256, cost192 = ((t192 + ncu - 1) / ncu) * 230;
  if (cost192 < cost256) return 3;
  return mixed_band_cols(p, ncu) > 0 ? 7 : 0;
}


template <int FA, int FB, int OUT, int LAY> static hipError_t launch_tile(const MmArgs& p, int tile, hipStream_t st) {
  switch (tile) {
    case 0: return launch_dma<FA, FB, 256, 256, 2, 4, 1, OUT, LAY>(p, st);
    case 3: return launch_dma<FA, FB, 256, 192, 2, 4, 1, OUT, LAY>(p, st);
    case 1: return launch_dma<FA, FB, 128, 128, 2, 2, 2, OUT, LAY>(p, st);
    case 5: return launch_dma<FA, FB, 64, 64, 1, 4, 2, OUT, LAY>(p, st);
    case 6: return launch_dma<FA, FB, 64, 64, 1, 4, 1, OUT, LAY, false, 8>(p, st);
    case 8: return launch_dma<FA, FB, 64, 32, 4, 1, 1, OUT, LAY, false, 8>(p, st);
    case 7: {
      const int64_t cb = mixed_band_cols(p, device_cu_count());
      if (cb > 0) return launch_mixed<FA, FB, OUT, LAY>(p, cb, st);
      return launch_dma<FA, FB, 256, 256, 2, 4, 1, OUT, LAY>(p, st);
    }
    default: return launch_dma<FA, FB, 64, 128, 1, 4, 2, OUT, LAY>(p, st);
  }
}

// The big-tile family for one format pair, output type and layout (operand
// extents below 2^31 bytes).  A mostly idle last round of 256 x 256 tiles
// becomes the 128 x 256 band of mm_fp8_mixed, in the same launch (as a
// second, small-tile launch it measured slower: 8192 x 6912 x 1536 98.4 us
// against 94.4 us for four rounds of 256 x 256).
template <int FA, int FB, int OUT, int LAY = 0> static hipError_t launch_dma_family(const MmArgs& p, hipStream_t st) {
  return launch_tile<FA, FB, OUT, LAY>(p, pick_tile(p, device_cu_count()), st);
}

// Short K (K <= kPreciseMaxK): the precise accumulation.  Its MFMA work is
// 8x, so the big tiles give way to 128 x 128 (two workgroups per CU).
static inline bool mm_precise(const MmArgs& p) { return p.K <= kPreciseMaxK; }
template <int FA, int FB, int OUT, int LAY> static hipError_t launch_dma_precise(const MmArgs& p, hipStream_t st) {
  switch (pick_tile(p, device_cu_count())) {
    case 5: return launch_dma<FA, FB, 64, 64, 1, 4, 2, OUT, LAY, true>(p, st);
    case 2: return launch_dma<FA, FB, 64, 128, 1, 4, 2, OUT, LAY, true>(p, st);
    default: return launch_dma<FA, FB, 128, 128, 2, 2, 2, OUT, LAY, true>(p, st);
  }
}

// Operand extents the 32-bit buffer offsets of the big-tile kernels cover.
static inline bool mm_fits31(const MmArgs& p) {
  const int64_t ea = (p.layout & 1) ? p.a_extent_km(0) : p.a_extent_from(0);
  const int64_t eb = (p.layout & 2) ? p.b_extent_km(0) : p.b_extent_from(0);
  return ea < (1ll << 31) && eb < (1ll << 31) && p.K < (1ll << 30);
}

}  // namespace fp8mi
