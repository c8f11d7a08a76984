// Device helpers shared by the libpkv kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;

// Native 16-byte vector (global_load/store_dwordx4).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16
// bf16 is the upper half of a binary32 pattern: widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 bf16 packed in a uint4 -> 8 floats, element order preserved.
__device__ __forceinline__ void unpack8(const u32x4 v, float* x) {
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
  x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
  x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// 8 fp16 packed in a u32x4 -> 8 floats (exact, subnormals included).
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ void unpack8_f16(const u32x4 v, float* x) {
  x[0] = f16_lo(v.x); x[1] = f16_hi(v.x);
  x[2] = f16_lo(v.y); x[3] = f16_hi(v.y);
  x[4] = f16_lo(v.z); x[5] = f16_hi(v.z);
  x[6] = f16_lo(v.w); x[7] = f16_hi(v.w);
}

// Widen 8 16-bit source elements: fp16 when kF16, else bf16.
template <bool kF16>
__device__ __forceinline__ void unpack8_src(const u32x4 v, float* x) {
  if constexpr (kF16) unpack8_f16(v, x); else unpack8(v, x);
}

// |x| as a binary32 bit pattern; for non-negative floats the unsigned
// integer order is the numeric order, so max-reductions run on integers.
__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7fffffffu; }

// ---------------------------------------------------------------- codecs
// OCP E4M3FN, round to nearest even, via the gfx950 packed converter.
// Exact (sign, subnormals, ties) for every |y| < 464; the store kernels only
// produce |y| <= 448 * (1 + 2^-8).  Element a lands in the lower byte of the
// selected 16-bit half.
template <bool kHighHalf>
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, kHighHalf);
}

// Four floats -> four E4M3 codes, element 0 in the lowest byte.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  return e4m3_pack2<true>(c, d, e4m3_pack2<false>(a, b, 0u));
}

// Exact decode of an E4M3 code (low byte of `code`) to binary32.
__device__ __forceinline__ float e4m3_decode(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// E2M1, round to nearest even with saturation at +-6, via the gfx950 scaled
// converter with unit scale (the scale contributes only its power-of-two
// exponent, so 1.0 leaves the value unchanged).  Exact for every non-NaN
// input.  Element a goes to the low nibble of byte kSel, element b to the
// high nibble.
template <int kSel>
__device__ __forceinline__ uint32_t e2m1_pack2(float a, float b, uint32_t old) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, kSel);
}

// ---------------------------------------------------------------- division
// binary32 x / s rounded to nearest even, given rs = RN(1/s): one product and
// Markstein's correction (P. Markstein, IBM J. Res. Dev. 34(1), 1990).  The
// residual x - q0*s is exact under fma and the corrected quotient is the
// correctly rounded one whenever no step under- or overflows; callers keep
// to that range (checked exhaustively over every significand pair on the
// host).  The sign is taken from x so that -0 stays -0.
__device__ __forceinline__ float div_by_scale(float x, float s, float rs) {
  const float q0 = x * rs;
  const float e = __builtin_fmaf(-q0, s, x);
  const float q1 = __builtin_fmaf(e, rs, q0);
  return __builtin_copysignf(q1, x);
}

// ---------------------------------------------------------------- lane ops
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xF, 0xF, false);
}
constexpr int kQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Max over aligned groups of kLanes lanes (power of two); every lane of the
// group receives the result.  All 64 lanes must be active.
template <int kLanes>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  if constexpr (kLanes >= 2) v = max(v, dpp<kQuadSwap1>(v));
  if constexpr (kLanes >= 4) v = max(v, dpp<kQuadSwap2>(v));
  if constexpr (kLanes >= 8) v = max(v, dpp<kRowHalfMirror>(v));
  if constexpr (kLanes >= 16) v = max(v, dpp<kRowMirror>(v));
  if constexpr (kLanes >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  if constexpr (kLanes >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}

// Orders the LDS accesses of one wave: what any lane wrote before the call
// is visible to every lane of the same wave after it (LDS operations of one
// wave execute in order; the fences keep the compiler from moving accesses
// across the call).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Value of a 64-bit variable held by lane `src` (all lanes must take part).
__device__ __forceinline__ int64_t lane_value(int64_t v, int src) {
  const int lo = __builtin_amdgcn_ds_bpermute(src << 2, (int)(uint32_t)v);
  const int hi = __builtin_amdgcn_ds_bpermute(src << 2, (int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int32_t t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
  return v;
}

// Streaming (read-once / write-once) 16-byte accesses.
__device__ __forceinline__ u32x4 load_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup b runs on
// XCD b % 8).  Renumbering b so that each XCD receives one contiguous range
// of logical blocks keeps neighbouring work items -- e.g. the tokens that
// share a cache page -- in one XCD's L2, where their partial-line writes
// merge.  A bijection on [0, gridDim.x) when gridDim.x is a multiple of 8.
constexpr uint32_t kNumXcd = 8;
__device__ __forceinline__ uint32_t xcd_contiguous_block() {
  const uint32_t b = blockIdx.x;
  return (b % kNumXcd) * (gridDim.x / kNumXcd) + b / kNumXcd;
}

// Division of n in [0, 2^31) by a divisor d in [1, 2^31) fixed for a launch,
// without a divide instruction: q = (n * m) >> (31 + l) with l = ceil(log2 d)
// and m = ceil(2^(31+l) / d).  Exact for every such n because
// 0 <= m*d - 2^(31+l) < d <= 2^l (T. Granlund and P. L. Montgomery,
// "Division by invariant integers using multiplication", PLDI 1994,
// Theorem 4.2 with N = 31).  m < 2^32 and n*m < 2^63.
struct FastDiv {
  uint32_t d;
  uint32_t m;
  uint32_t shift;  // 31 + l
  __host__ __device__ static FastDiv make(uint32_t divisor) {
    FastDiv f;
    f.d = divisor;
    uint32_t l = 0;
    while ((1ull << l) < divisor) ++l;
    f.shift = 31 + l;
    f.m = (uint32_t)(((1ull << (31 + l)) + divisor - 1) / divisor);
    return f;
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    return (uint32_t)(((uint64_t)n * m) >> shift);
  }
};

// slot -> (page, offset) for a block size that may or may not be a power of two.
__device__ __forceinline__ void split_slot(int64_t slot, int32_t block_size, int32_t log2_bs,
                                           int64_t& page, int64_t& off) {
  if (log2_bs >= 0) {
    page = slot >> log2_bs;
    off = slot & (int64_t)(block_size - 1);
  } else {
    page = slot / block_size;
    off = slot - page * block_size;
  }
}

}  // namespace pkv
