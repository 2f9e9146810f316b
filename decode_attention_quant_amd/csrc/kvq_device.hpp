// kvq_device.hpp -- device helpers for gfx950: vector types and the element
// and scale codecs shared by the kernels.
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
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

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

}  // namespace kvq
