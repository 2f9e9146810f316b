// kvq_device.hpp -- device helpers for gfx950: element codecs, lane
// exchanges and the fixed-order 256-point Hadamard butterfly.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_format.hpp"

namespace kvq {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& f) {
  static_assert(sizeof(To) == sizeof(From), "size");
  To t;
  __builtin_memcpy(&t, &f, sizeof(To));
  return t;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// ----------------------------------------------------------------- encoders
// All of these are exact, deterministic definitions (round to nearest even,
// saturating), matching the format definitions of the KV formats.

// IEEE fp32 -> fp16 bits, RNE, overflow -> inf (BF16-format V plane).
__device__ __forceinline__ uint32_t f16_bits(float x) { return bitcast<uint16_t>((_Float16)x); }

// Non-negative scale -> fp16 bits, RNE, saturating at 65504.
__device__ __forceinline__ uint32_t f16_scale_bits(float s) { return f16_bits(fminf(s, 65504.0f)); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) { return (float)bitcast<_Float16>((uint16_t)b); }

// fp32 -> E4M3FN code: RNE, saturating at +-448, sign kept (-0 -> 0x80).
// v_cvt_pk_fp8_f32 rounds to nearest even over the whole E4M3 grid
// (subnormals included) but turns values past the 464 midpoint into NaN,
// so the input is clamped first.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  x = fmaxf(fminf(x, 448.0f), -448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false) & 0xFFu;
}

// E4M3FN code -> fp32 (exact; 0x7F/0xFF give NaN).
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)code, false)[0];
}

// fp32 -> E2M1 code, RNE with ties to the even code, saturating at +-6.
// The grid {0, .5, 1, 1.5, 2, 3, 4, 6} has midpoints .25 .75 1.25 1.75 2.5
// 3.5 5; a midpoint goes up exactly when the upper neighbour's code is even.
__device__ __forceinline__ uint32_t e2m1_code(float x) {
  const float a = fabsf(x);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return c | (__float_as_uint(x) >> 31 << 3);
}

// ----------------------------------------------------------------- lanes

// xor-shuffle within groups of 16 lanes (partner = lane ^ m, m < 16)
__device__ __forceinline__ float shfl_xor16(float v, int m) { return __shfl_xor(v, m, 16); }

// ----------------------------------------------------------------- FWHT
// Fixed-order 256-point normalized Hadamard transform for one row held by
// 16 lanes x 16 values (lane j holds elements 16j .. 16j+15).  Stages run
// for h = 1, 2, ..., 128 in that order; each butterfly is one fp32 add or
// subtract:  (y_i, y_{i+h}) <- (y_i + y_{i+h}, y_i - y_{i+h})  for i with
// bit h clear, and the result is scaled by 2^-4 (exact).  The encoders use
// this order as part of the format (NInfer guide: 256-point normalized
// Hadamard before INT8 K and NVFP4 K/V quantization).
__device__ __forceinline__ void fwht256_rows16(float (&x)[16], int lane16) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    const bool upper = (lane16 & m) != 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = shfl_xor16(x[i], m);
      x[i] = upper ? (p - x[i]) : (x[i] + p);
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] *= 0.0625f;
}

}  // namespace kvq
