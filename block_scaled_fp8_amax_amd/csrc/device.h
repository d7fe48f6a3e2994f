// Device helpers shared by the fp8blk HIP kernels (gfx950 only).
//
// Numeric building blocks:
//   * bf16 <-> fp32: widening is a shift; narrowing uses the gfx950
//     v_cvt_pk_bf16_f32 instruction (round to nearest even).
//   * fp32 -> e4m3fn: v_cvt_pk_fp8_f32 rounds to nearest even and keeps the
//     sign of zero, but maps magnitudes above 464 to NaN (0x7F); callers
//     whose values can exceed 448 clamp first.
//   * block amax on bf16 bit patterns: the 15 magnitude bits of a finite
//     bf16 order like the values, so an integer max is exact.
//   * the correctly rounded quotient RN32(x / s) from a correctly rounded
//     reciprocal y = RN32(1 / s) and two fused multiply-adds
//     (Markstein's correction): q0 = RN(x*y), r = x - q0*s (exact),
//     q = RN(q0 + r*y).  Blocks with amax < 2^-60 are pre-scaled by 2^64 so
//     that the remainder never underflows; an exhaustive sweep over every
//     bf16 pair (x, amax) found no input whose e4m3 code differs from the
//     one the IEEE quotient gives.  The remainder is formed negated,
//     -r = RN(q0*s - x), and applied as q = RN((-r)*(-y) + q0): for x != 0
//     that is the same exact value, so the same rounding, and for x = -0 it
//     keeps the sign (-r = +0, and (+0)*(-y) + (-0) = -0), where the plain
//     form gives +0; so no separate sign fix is needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> one dword of two bf16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  v2f v = {lo, hi};
  v2bf r = __builtin_convertvector(v, v2bf);
  return __builtin_bit_cast(uint32_t, r);
}

// Largest bf16 magnitude (15-bit pattern) among the 2*N values of N dwords.
template <int N>
__device__ __forceinline__ uint32_t absmax_bits(const uint32_t* w) {
  v2u16 m = __builtin_bit_cast(v2u16, w[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int i = 1; i < N; ++i) {
    v2u16 t = __builtin_bit_cast(v2u16, w[i] & 0x7FFF7FFFu);
    m = __builtin_elementwise_max(m, t);
  }
  return m[0] > m[1] ? (uint32_t)m[0] : (uint32_t)m[1];
}

// DPP lane permutations (gfx9 encodings).
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i within each 16 lanes

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
  return v > o ? v : o;
}

// Max over aligned groups of LANES consecutive lanes (LANES = 4 or 16);
// every lane of the group receives the result.  All lanes must be active.
template <int LANES>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  static_assert(LANES == 4 || LANES == 16, "group size");
  v = dpp_max<kQuadSwap1>(v);
  v = dpp_max<kQuadSwap2>(v);
  if constexpr (LANES == 16) {
    v = dpp_max<kRowHalfMirror>(v);
    v = dpp_max<kRowMirror>(v);
  }
  return v;
}

// Max over the whole wave (64 lanes), wave-uniform result.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = group_max<16>(v);
  uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  a = a > b ? a : b;
  c = c > d ? c : d;
  return a > c ? a : c;
}

// ---------------------------------------------------------------- fp32 scale

// Per-block constants of the fp32-scale path.
struct F32Block {
  float s;    // stored scale RN32(amax / 448)
  float sp;   // s * pre (exact)
  float y;    // RN32(1 / sp); 0 for an all-zero block
  float pre;  // 1 or 2^64
};

__device__ __forceinline__ F32Block f32_block(uint32_t amax_bits) {
  F32Block b;
  float amax = __uint_as_float(amax_bits << 16);
  b.s = amax / kE4M3Max;                      // IEEE division, correctly rounded
  b.pre = amax < 0x1p-60f ? 0x1p64f : 1.0f;
  b.sp = b.s * b.pre;
  b.y = amax_bits == 0 ? 0.0f : 1.0f / b.sp;  // IEEE division
  return b;
}

// RN32(x / s) with the sign of x (also for x = -0: x*pre, q0 and q keep
// it, and the negated remainder is +0).
__device__ __forceinline__ float f32_quot(float x, const F32Block& b) {
  float xp = x * b.pre;
  float q0 = xp * b.y;
  float rn = __builtin_fmaf(q0, b.sp, -xp);   // -r, exact
  return __builtin_fmaf(rn, -b.y, q0);
}

// f32_quot for a block whose prescale is 1 (amax >= 2^-60): the same
// operations without the multiplications by 1.
__device__ __forceinline__ float f32_quot_unit(float x, const F32Block& b) {
  float q0 = x * b.y;
  float rn = __builtin_fmaf(q0, b.sp, -x);    // -r, exact
  return __builtin_fmaf(rn, -b.y, q0);
}

// ---------------------------------------------------------------- E8M0 scale

// E8M0 code of a block from its bf16 amax bit pattern.
//   CEIL : X = smallest integer with amax <= 448 * 2^X.  With amax =
//          (1 + m/128) * 2^(E-127) and 448 = 1.75 * 2^8 this is
//          E - 135 + [m > 0x60] (0x60 = mantissa of 1.75), code = X + 127.
//   FLOOR: X = floor(log2 amax) - 8 = E - 135, code = E - 8.
// Both clamp the code to [0, 254]; subnormal and zero amax give code 0.
template <bool FLOOR>
__device__ __forceinline__ uint32_t e8m0_code(uint32_t amax_bits) {
  int e = (int)(amax_bits >> 7);
  int c = FLOOR ? e - 8 : e - 8 + ((amax_bits & 0x7F) > 0x60 ? 1 : 0);
  c = c < 0 ? 0 : c;
  c = c > 254 ? 254 : c;
  return (uint32_t)c;
}

// 2^-X = 2^(127 - code) as an fp32 (code <= 247 for finite bf16 input, so
// the result is a normal number).
__device__ __forceinline__ float e8m0_inv(uint32_t code) {
  return __uint_as_float((254u - code) << 23);
}

// 2^X = 2^(code - 127) as an fp32 (code 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_val(uint32_t code) {
  return code == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(code << 23);
}

// ------------------------------------------------------------- code stores

// Codes that fit in half the 256 MiB Infinity Cache are written with
// ordinary stores, so that the GEMM that usually consumes them next finds
// them cached; larger outputs (a whole layer's prequant) stream past the
// caches with nontemporal stores.
constexpr int64_t kCachedCodeBytes = int64_t(128) << 20;

template <bool CACHED, typename T>
__device__ __forceinline__ void store_code(T v, T* p) {
  if constexpr (CACHED)
    *p = v;
  else
    __builtin_nontemporal_store(v, p);
}

// ----------------------------------------------------------- e4m3 packing

// Four fp32 -> four e4m3fn codes in one dword (byte i = value i).
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)r, true);
}

__device__ __forceinline__ float clamp448(float v) {
  return __builtin_fminf(__builtin_fmaxf(v, -kE4M3Max), kE4M3Max);
}

// Decode four e4m3fn codes of a dword to fp32 (exact).
__device__ __forceinline__ void decode4_e4m3(uint32_t w, float* out) {
  v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

}  // namespace fp8blk
