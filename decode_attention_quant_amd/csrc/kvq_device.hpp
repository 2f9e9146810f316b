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

// ----------------------------------------------------------- DPP lane exchange

constexpr int QUAD_XOR1 = 0xB1;  // DPP quad_perm [1, 0, 3, 2]
constexpr int QUAD_XOR2 = 0x4E;  // DPP quad_perm [2, 3, 0, 1]
constexpr int ROW_SHL4 = 0x104;  // lane i reads lane i + 4 of its row of 16
constexpr int ROW_SHR4 = 0x114;  // lane i reads lane i - 4
constexpr int ROW_ROR8 = 0x128;  // lane i reads lane (i + 8) mod 16

// Every lane is written (full row and bank masks), so the move needs no
// "old" value: mov_dpp leaves it undefined, where update_dpp with an old of
// 0 would first put a zero into the destination, one more instruction per
// exchange.
template <int CTRL>
__device__ __forceinline__ float quad_swap(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// The value of lane (i ^ M) of the same row of 16 lanes, M in {1, 2, 4, 8}.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (M == 1) return quad_swap<QUAD_XOR1>(v);
  else if constexpr (M == 2) return quad_swap<QUAD_XOR2>(v);
  else if constexpr (M == 8) return quad_swap<ROW_ROR8>(v);
  else {
    static_assert(M == 4, "");
    // lanes 0-3 and 8-11 (banks 0, 2) read i + 4; lanes 4-7 and 12-15 read i - 4
    // (banks 1 and 3 of the first move are left undefined and overwritten)
    const int lo = __builtin_amdgcn_mov_dpp(__float_as_int(v), ROW_SHL4, 0xF, 0x5, false);
    return __int_as_float(__builtin_amdgcn_update_dpp(lo, __float_as_int(v), ROW_SHR4, 0xF, 0xA, false));
  }
}

template <int M>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v) {
  return __float_as_uint(lane_xor<M>(__uint_as_float(v)));
}

// One butterfly stage across lanes M apart: the lower lane of each pair
// keeps x + partner and the upper one partner - x, each rounded once.
// M <= 8 is a DPP permutation inside a row of 16 lanes; M = 16 and 32 use
// the swap instructions, which leave the lower lane's value in result 0
// and the upper lane's in result 1, in both lanes of the pair.
template <int M>
__device__ __forceinline__ float xlane_butterfly(float x, int lane) {
  const float sg = (lane & M) ? -1.0f : 1.0f;
  if constexpr (M <= 8) {
    return __builtin_fmaf(sg, x, lane_xor<M>(x));
  } else {
    static_assert(M == 16 || M == 32, "");
    const uint32_t v = bitcast<uint32_t>(x);
    const auto s = M == 16 ? __builtin_amdgcn_permlane16_swap(v, v, false, false)
                           : __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __builtin_fmaf(sg, bitcast<float>((uint32_t)s[1]), bitcast<float>((uint32_t)s[0]));
  }
}

}  // namespace kvq
