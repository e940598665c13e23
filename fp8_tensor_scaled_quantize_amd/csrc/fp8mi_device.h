// Device-side building blocks shared by the quantize, fold and GEMM kernels:
// fp8 encode, bf16 rounding, wave/block reductions and the ring fold.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8mi {

enum Fmt : int { kE4M3 = 0, kE5M2 = 1 };
enum Dtype : int { kF32 = 0, kF16 = 1, kBF16 = 2, kFp8E4M3 = 3, kFp8E5M2 = 4 };

template <int FMT> struct FmtTraits;
// OCP E4M3FN: largest finite 448 (S.1111.110); E5M2: 57344 (S.11110.11).
template <> struct FmtTraits<kE4M3> { static constexpr float kMax = 448.0f; };
template <> struct FmtTraits<kE5M2> { static constexpr float kMax = 57344.0f; };

// ---------------------------------------------------------------------------
// Input element types, widened exactly to fp32.
// ---------------------------------------------------------------------------
template <int DT> struct In;
template <> struct In<kF32> { using T = float; static constexpr int kBytes = 4; };
template <> struct In<kF16> { using T = uint16_t; static constexpr int kBytes = 2; };
template <> struct In<kBF16> { using T = uint16_t; static constexpr int kBytes = 2; };

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
  return (float)v;  // exact (v_cvt_f32_f16)
}

// Element widening from a 32-bit word holding two 16-bit values (lo = first).
template <int DT> __device__ __forceinline__ void widen2(uint32_t w, float& a, float& b) {
  if constexpr (DT == kBF16) {
    a = __uint_as_float(w << 16);
    b = __uint_as_float(w & 0xFFFF0000u);
  } else {
    a = f16_to_f32(w & 0xFFFFu);
    b = f16_to_f32(w >> 16);
  }
}

// Load one element (any alignment of its own size).
template <int DT> __device__ __forceinline__ float load1(const void* base, int64_t idx) {
  if constexpr (DT == kF32) return static_cast<const float*>(base)[idx];
  else if constexpr (DT == kBF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[idx]);
  else return f16_to_f32(static_cast<const uint16_t*>(base)[idx]);
}

// ---------------------------------------------------------------------------
// fp8 encode.  The fast path clamps to +-fmt_max with v_med3 and converts with
// v_cvt_pk_{fp8,bf8}_f32 (round to nearest even; exact for every non-NaN fp32
// input once clamped).  NaN inputs take enc_exact, which gives the NaN code
// 0x7F with the input's sign.
// ---------------------------------------------------------------------------
template <int FMT> __device__ __forceinline__ float clampf(float v) {
  constexpr float m = FmtTraits<FMT>::kMax;
  return __builtin_amdgcn_fmed3f(v, -m, m);
}

// Four values -> one word, element j in byte j.
template <int FMT> __device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int w;
  if constexpr (FMT == kE4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clampf<FMT>(a), clampf<FMT>(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clampf<FMT>(c), clampf<FMT>(d), w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(clampf<FMT>(a), clampf<FMT>(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(clampf<FMT>(c), clampf<FMT>(d), w, true);
  }
  return (uint32_t)w;
}

// The same conversion without the clamp, for values already within
// +-fmt_max (the conversion rounds those exactly).
template <int FMT> __device__ __forceinline__ uint32_t cvt4_inrange(float a, float b, float c, float d) {
  int w;
  if constexpr (FMT == kE4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

// Integer saturating round-to-nearest-even encoder, used for words that hold
// a NaN.  Normal range: drop the low fp32 mantissa bits with RNE (a carry
// moves into the exponent field exactly as the format's code order does);
// subnormal range: the code is the value in units of the smallest subnormal,
// rounded to nearest even.
template <int FMT> __device__ __forceinline__ uint32_t enc_exact(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t s = (u >> 24) & 0x80u, a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu | s;
  if constexpr (FMT == kE4M3) {
    if (a >= 0x43E00000u) return 0x7Eu | s;                  // >= 448
    if (a < 0x3C800000u)                                     // < 2^-6
      return (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f) | s;
    uint32_t c = (a >> 20) - (120u << 3);
    const uint32_t rem = a & 0xFFFFFu;
    c += (rem > 0x80000u) || (rem == 0x80000u && (c & 1u));
    return c | s;
  } else {
    if (a >= 0x47600000u) return 0x7Bu | s;                  // >= 57344
    if (a < 0x38800000u)                                     // < 2^-14
      return (uint32_t)__builtin_rintf(__uint_as_float(a) * 65536.0f) | s;
    uint32_t c = (a >> 21) - (112u << 2);
    const uint32_t rem = a & 0x1FFFFFu;
    c += (rem > 0x100000u) || (rem == 0x100000u && (c & 1u));
    return c | s;
  }
}

template <int FMT> __device__ __forceinline__ uint32_t enc4_exact(float a, float b, float c, float d) {
  return enc_exact<FMT>(a) | (enc_exact<FMT>(b) << 8) | (enc_exact<FMT>(c) << 16) | (enc_exact<FMT>(d) << 24);
}

// A scale s for which x * s is NaN only where x is NaN: finite and nonzero.
// With any other scale (0, +-inf, NaN) 0 * inf or inf * 0 makes a NaN out of
// a non-NaN input, so the kernels send every element to enc_exact, which
// encodes the product itself; the NaN test on the raw input that picks the
// fast conversion is valid only for a regular scale.
__device__ __forceinline__ bool scale_regular(float s) {
  return s != 0.0f && __builtin_fabsf(s) <= 3.40282347e38f;
}

// ---------------------------------------------------------------------------
// bf16 round to nearest even from fp32 (overflow to inf, NaN kept quiet).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  // both results, then a select: written with an early return for NaN, the
  // compiler emitted an exec-mask branch per value, which made the GEMM's
  // 128-value-per-lane epilogue take ~5 µs
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet_nan = ((u >> 16) | 0x40u) & 0xFFFFu;
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? quiet_nan : rounded;
}

// Four fp32 -> bf16, round to nearest even, packed two per word, by the
// hardware conversion (v_cvt_pk_bf16_f32).  Checked on MI355X against
// f32_to_bf16_rne over all 2^32 fp32 inputs: the same bits for every non-NaN
// input (denormals and overflow to infinity included), a NaN for every NaN
// (its payload may differ).
__device__ __forceinline__ uint2 bf16x4_rne(float a, float b, float c, float d) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const f32x2 lo = {a, b}, hi = {c, d};
  return make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2)),
                    __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2)));
}

// ---------------------------------------------------------------------------
// Reductions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Max over the block; the result is valid in every thread.  `red` holds one
// float per wave.
template <int NT> __device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// The published scale for a window maximum m: fmt_max / m (IEEE division),
// or 1.0 when m is 0 or not finite, or the quotient is not a finite positive
// number.
// ---------------------------------------------------------------------------
template <int FMT> __device__ __forceinline__ float scale_from_max(float m) {
  float s = 1.0f;
  if (m > 0.0f && m <= 3.40282347e38f) {
    const float q = FmtTraits<FMT>::kMax / m;
    if (q > 0.0f && q <= 3.40282347e38f) s = q;
  }
  return s;
}

// ---------------------------------------------------------------------------
// Ring fold, executed by one full wave (64 lanes): amax = v (REDUCE false,
// the same value in every lane) or the maximum of the lanes' v (REDUCE
// true); write amax into hist[slot], advance the slot modulo H,
// publish fmt_max / max(hist) (1.0 when that maximum is 0 or not finite, or
// the quotient is not a finite positive number).  The slot index and the
// first 64 history entries are loaded before anything waits, so they travel
// together with whatever loads the caller left in flight for v (one memory
// round trip instead of two or three).  The maximum of the new window
// is max(amax, hist[i] for i != slot), which is exact in any order.
// ---------------------------------------------------------------------------
template <int FMT, bool REDUCE = false>
__device__ void ring_fold_wave(uint32_t* ring, int H, float v, float* scale_inv_out, float s_used, float* amax_out) {
  const int lane = threadIdx.x & 63;
  const float* hist = reinterpret_cast<const float*>(ring);
  // unconditional loads (lanes at or past H re-read entry 0, unused), so no
  // branch separates them and neither waits for the other
  const float h0 = hist[lane < H ? lane : 0];
  const uint32_t slot_word = ring[H + 1];
  const float amax = REDUCE ? wave_max(v) : v;
  const uint32_t slot = slot_word % (uint32_t)H;
  float m = amax;
  if (lane < H && (uint32_t)lane != slot) m = fmaxf(m, h0);
  for (int i = lane + 64; i < H; i += 64)
    if ((uint32_t)i != slot) m = fmaxf(m, hist[i]);
  m = wave_max(m);
  if (lane == 0) {
    const float s = scale_from_max<FMT>(m);
    reinterpret_cast<float*>(ring)[slot] = amax;
    ring[H] = __float_as_uint(s);
    ring[H + 1] = (slot + 1u == (uint32_t)H) ? 0u : slot + 1u;
    if (scale_inv_out) *scale_inv_out = 1.0f / s_used;
    if (amax_out) *amax_out = amax;
  }
}

// ---------------------------------------------------------------------------
// Cross-workgroup amax publication.
//
// Device-scope atomics to one address serialise across the XCDs (about 12 ns
// each on MI355X), so workgroups spread their partial amax over kFoldSlots
// slots on separate 128-byte lines of the ring's scratch region: a workgroup
// maxes its amax into slot (id % nslot) and takes that slot's ticket; the
// last member of each slot takes the completion ticket; the workgroup that
// takes the last completion ticket reduces the slots, folds, and clears the
// scratch.  Ordering rests on returning device-scope atomics: every atomic
// below returns its old value, and a workgroup waits for each to come back
// (s_waitcnt on the vector memory counter, which the wave's operations
// decrement in issue order) before issuing the next, so its partial amax is
// performed at the device's coherence point before its ticket is; the slot
// and completion tickets are totally ordered per address, and the final
// reads are device-scope atomic loads.  No L2 write-back fence is needed
// because no plain store is read by another workgroup.
// ---------------------------------------------------------------------------
constexpr int kFoldSlots = 32;
constexpr int kFoldSlotStride = 32;  // words: 128 bytes between slots
static_assert(kFoldSlots * kFoldSlotStride == 1024, "ring scratch is FP8MI_RING_SCRATCH_WORDS words");

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector memory operations of this wave are outstanding.
template <int N> __device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t dev_load(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t dev_max(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t dev_add(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t dev_xchg(uint32_t* p, uint32_t v) {
  return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Max a non-negative fp32 into a word holding fp32 bits; skips the
// read-modify-write when the word already holds at least as much.
__device__ __forceinline__ void publish_max(uint32_t* p, float v) {
  const uint32_t bits = __float_as_uint(v);
  if (bits > dev_load(p)) {
    const uint32_t old = dev_max(p, bits);
    asm volatile("" ::"v"(old));  // keep the returning form of the atomic
  }
  wait_vmem();
}

// First half of a workgroup's ring protocol, thread 0 only: max the block's
// amax into its slot.  The atomic is left in flight (its old value returned
// for ring_block_finish to consume), so a kernel that knows its amax before
// storing its codes can publish it first and let the round trip overlap the
// stores.  The library is built without the compiler's atomic optimizer,
// which would turn this one-lane atomic into a wave reduction that needs the
// returned value at once.
__device__ __forceinline__ uint32_t ring_publish(uint32_t* ring, int H, float block_amax) {
  const uint32_t nblk = gridDim.x * gridDim.y * gridDim.z;
  const uint32_t nslot = nblk < (uint32_t)kFoldSlots ? nblk : (uint32_t)kFoldSlots;
  const uint32_t bid = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  return dev_max(ring + H + 4 + (bid % nslot) * kFoldSlotStride, __float_as_uint(block_amax));
}

// Second half; every thread of the block calls it, thread 0 with the value
// ring_publish returned.  Thread 0 waits for its published maximum to come
// back, takes the slot's ticket, and the last member of a slot the
// completion ticket.  `flag` is one word of LDS that no thread reads between
// the caller's last barrier and this call.
template <int FMT>
__device__ void ring_block_finish(uint32_t* ring, int H, uint32_t published, float s_used, float* scale_inv_out,
                                  float* amax_out, uint32_t* flag) {
  const uint32_t nblk = gridDim.x * gridDim.y * gridDim.z;
  const uint32_t nslot = nblk < (uint32_t)kFoldSlots ? nblk : (uint32_t)kFoldSlots;
  uint32_t* scratch = ring + H + 4;
  if (threadIdx.x == 0) {
    // the slot's atomic must have come back: the compiler waits for its value
    // here (a wave's vector memory operations complete in issue order, so
    // stores issued after the atomic may stay in flight -- the fold reads
    // none of them)
    asm volatile("" ::"v"(published) : "memory");
    const uint32_t bid = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const uint32_t slot = bid % nslot;
    const uint32_t members = nblk / nslot + (slot < nblk % nslot ? 1u : 0u);
    bool last = dev_add(scratch + slot * kFoldSlotStride + 1, 1u) == members - 1u;
    if (last) last = dev_add(ring + H + 2, 1u) == nslot - 1u;
    *flag = last ? 1u : 0u;
  }
  __syncthreads();
  if (*flag == 0u || threadIdx.x >= 64) return;
  // The last workgroup: wave 0 reduces the slots, folds, clears the scratch.
  const int lane = threadIdx.x;
  // the slot reads stay in flight while the fold issues its history loads
  const float a = (uint32_t)lane < nslot ? __uint_as_float(dev_load(scratch + lane * kFoldSlotStride)) : 0.0f;
  ring_fold_wave<FMT, true>(ring, H, a, scale_inv_out, s_used, amax_out);
  if ((uint32_t)lane < nslot) {
    (void)dev_xchg(scratch + lane * kFoldSlotStride, 0u);
    (void)dev_xchg(scratch + lane * kFoldSlotStride + 1, 0u);
  }
  if (lane == 0) (void)dev_xchg(ring + H + 2, 0u);
}

// End of a ring-mode quantize workgroup (both halves at once); every thread
// of the block calls it with the block's amax.  `flag` is one word of LDS.
template <int FMT>
__device__ void ring_block_done(uint32_t* ring, int H, float block_amax, float s_used, float* scale_inv_out,
                                float* amax_out, uint32_t* flag) {
  const uint32_t published = threadIdx.x == 0 ? ring_publish(ring, H, block_amax) : 0u;
  ring_block_finish<FMT>(ring, H, published, s_used, scale_inv_out, amax_out, flag);
}

}  // namespace fp8mi
