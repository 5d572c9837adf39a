// Shared device helpers of the MoE-layer kernels (gfx950 / CDNA4).
#pragma once
#include <utility>
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

// fn.template operator()<I>() for I = 0 .. N-1, expanded at compile time (register arrays
// indexed by I stay in registers however large the body is).
template <int N, class Fn>
MOE_DEV void static_for(Fn&& fn) {
  [&]<int... I>(std::integer_sequence<int, I...>) { (fn.template operator()<I>(), ...); }(
      std::make_integer_sequence<int, N>{});
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

namespace moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16

MOE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float32 -> bfloat16, round to nearest, ties to even (inputs are finite).
MOE_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------- MXFP8 scalar pieces
//
// MXFP8 (OCP MX v1.0): e4m3 elements, one e8m0 exponent byte per 32 values.  A
// block's exponent is floor(log2 amax) - 8, clamped to [-127, 127], stored
// biased by 127.  For a float32 amax with biased exponent field ef that byte is
// max(ef - 8, 0): ef = 0 covers both amax == 0 and subnormal amax, whose true
// exponent is below -127 and clamps.

MOE_DEV uint32_t e8m0_from_amax(float amax) {
  int ef = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return (uint32_t)max(ef - 8, 0);
}

// 2^(127 - byte) as a float: the factor that maps a block into e4m3 range.
MOE_DEV float e8m0_inv_scale(uint32_t byte) { return __uint_as_float((254u - byte) << 23); }

// 2^(byte - 127) as a float (byte >= 1; byte 0 is only used with zero codes).
MOE_DEV float e8m0_scale(uint32_t byte) {
  return byte ? __uint_as_float(byte << 23) : __uint_as_float(0x00400000u);
}

MOE_DEV float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// Four already-scaled values -> four e4m3 codes (round to nearest even) in one word.
// The conversion instruction does not saturate, so values are clamped first.
// The first conversion writes the low half of its destination and keeps the high half, which
// the second one overwrites: any value serves as the first's "old" word, so the clamped input
// itself is passed (no register has to be zeroed).
MOE_DEV uint32_t pack4_e4m3(float a, float b, float c, float d) {
  const float ca = clamp448(a);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(ca, clamp448(b), __float_as_int(ca), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), w, true);
  return (uint32_t)w;
}

// e4m3 code -> float (used by the requantisation kernels).
MOE_DEV float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 0xFu;
  uint32_t m = c & 0x7u;
  float v;
  if (e == 0) {
    v = (float)m * 0.001953125f;  // m * 2^-9
  } else {
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) * 2^(e-7)
  }
  return __uint_as_float(__float_as_uint(v) | s);
}

// ---------------------------------------------------------------- wave reductions

template <int W>
MOE_DEV float group_max(float v) {  // max over aligned groups of W lanes (W power of 2, <= 64)
#pragma unroll
  for (int o = 1; o < W; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, W));
  return v;
}

// Maximum over each aligned group of 32 lanes, without the LDS crossbar: row rotations by 8, 4,
// 2 and 1 (DPP) leave every lane of a 16-lane row with the row maximum, then v_permlane16_swap
// exchanges the maxima of the two rows of each 32-lane half.
MOE_DEV float group_max32(float v) {
  // v >= 0: non-negative floats order like their bit patterns, so the maximum is taken on the
  // integers (a float maximum of values that crossed lanes as integers is preceded by a
  // canonicalising instruction each time)
  uint32_t u = __float_as_uint(v);
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x128, 0xF, 0xF, false));
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x124, 0xF, 0xF, false));
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x122, 0xF, 0xF, false));
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x121, 0xF, 0xF, false));
  const auto pr = __builtin_amdgcn_permlane16_swap((int)u, (int)u, false, false);
  return __uint_as_float(max((uint32_t)pr[0], (uint32_t)pr[1]));
}

template <int W>
MOE_DEV float group_sum(float v) {  // fixed-order butterfly: same result on every run
#pragma unroll
  for (int o = 1; o < W; o <<= 1) v += __shfl_xor(v, o, W);
  return v;
}

MOE_DEV int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace moe
