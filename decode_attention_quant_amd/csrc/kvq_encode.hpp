// kvq_encode.hpp -- the row encoders of the write path, shared by the
// quantize-append kernel and the fused decode step.
//
// K rows: the 4 lanes of a quad encode one token's row, lane q holding
// elements [q E, (q + 1) E), E = D / 4.  Scale groups of 16, 32 and 64
// values lie inside one lane; the row-wide FP8 scale is reduced over the
// quad; the rotation runs stages h = 1 .. 32 inside a lane and h = 64, 128
// across the quad.  The K tile keeps one token's values together, so each
// lane stores whole 8- or 16-byte pieces.
//
// V rows: each row of 16 lanes holds 4 consecutive tokens, lane j holding
// elements [j F, (j + 1) F), F = D / 16, of all 4.  The V tile interleaves
// 4 consecutive slots (a slab) inside every 32-bit word, so when the 4
// tokens fill one slab (consecutive slots, the first a multiple of 4) each
// lane writes whole words: 8-bit codes after a 4 x 4 word transpose across
// the quad, 4-bit codes (one column of a token pair per byte) after an
// 8 x 8 word transpose across 8 lanes.  Otherwise 8- and 16-bit codes are
// written token by token (two partial writes per word for consecutive
// slots that straddle two slabs), and 4-bit codes nibble by nibble with
// atomic and/or, which keeps the other token of the pair intact.  The
// rotation runs stages h = 1 .. 8 inside a lane and h = 16 .. 128 across
// lanes (xor 1, 2, 4, 8).
//
// Every cross-lane step is a DPP permutation, and every rotation stage
// rounds exactly like the fixed butterfly order of the format.
#pragma once
#include <hip/hip_runtime.h>

#include "kvq_device.hpp"
#include "kvq_internal.hpp"

namespace kvq {
namespace enc {


// Lanes c = 0 .. 3 of a quad hold W[0 .. 3]; afterwards lane c holds
// element c of every lane: W[k] = (W of lane k)[c].  Two butterfly stages,
// over lane bit 0 and lane bit 1, each swapping the elements whose index bit
// differs from the lane's.
__device__ __forceinline__ void quad_transpose(uint32_t (&W)[4], int c) {
  {
    const bool odd = c & 1;
    const uint32_t r0 = lane_xor_u32<1>(odd ? W[0] : W[1]), r1 = lane_xor_u32<1>(odd ? W[2] : W[3]);
    W[0] = odd ? r0 : W[0];
    W[1] = odd ? W[1] : r0;
    W[2] = odd ? r1 : W[2];
    W[3] = odd ? W[3] : r1;
  }
  {
    const bool hi = c & 2;
    const uint32_t r0 = lane_xor_u32<2>(hi ? W[0] : W[2]), r1 = lane_xor_u32<2>(hi ? W[1] : W[3]);
    W[0] = hi ? r0 : W[0];
    W[1] = hi ? r1 : W[1];
    W[2] = hi ? W[2] : r0;
    W[3] = hi ? W[3] : r1;
  }
}

// Lanes c = 0 .. 7 of a group of 8 hold W[0 .. 7]; afterwards lane c holds
// element c of every lane of the group: W[k] = (W of lane k)[c].  Stage M
// (1, 2, 4) swaps element i + M of the lower lane of each pair with element
// i of the upper one (bit M of i clear).
template <int M>
__device__ __forceinline__ void oct_stage(uint32_t (&W)[8], int c) {
  const bool up = (c & M) != 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i & M) continue;
    const uint32_t r = lane_xor_u32<M>(up ? W[i] : W[i + M]);
    if (up) W[i] = r;
    else W[i + M] = r;
  }
}

__device__ __forceinline__ void oct_transpose(uint32_t (&W)[8], int c) {
  oct_stage<1>(W, c);
  oct_stage<2>(W, c);
  oct_stage<4>(W, c);
}

// Max over the L lanes (L a power of two <= 16) whose index differs only in
// its low log2 L bits.
template <int L>
__device__ __forceinline__ float max_over_lanes(float a) {
  if constexpr (L >= 2) a = fmaxf(a, lane_xor<1>(a));
  if constexpr (L >= 4) a = fmaxf(a, lane_xor<2>(a));
  if constexpr (L >= 8) a = fmaxf(a, lane_xor<4>(a));
  if constexpr (L >= 16) a = fmaxf(a, lane_xor<8>(a));
  return a;
}

// Fixed-order FWHT-256 scaled by 2^-4 (NInfer guide: normalized 256-point
// Hadamard before INT8 K and NVFP4 K/V quantization) of one row held by a
// quad, lane q holding elements 64 q .. 64 q + 63.  Stage h pairs element i
// with i + h (bit h of i clear) into (y_i + y_{i+h}, y_i - y_{i+h}), one
// fp32 rounding each; across lanes the lower lane of a pair keeps the sum
// and the upper one the difference, both as fma(+-1, own, partner), which
// rounds p + x or p - x once.
__device__ __forceinline__ void fwht256_quad(float (&x)[64], int q) {
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
  {
    const float sg = (q & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] = __builtin_fmaf(sg, x[i], quad_swap<QUAD_XOR1>(x[i]));
  }
  {
    const float sg = (q & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] = __builtin_fmaf(sg, x[i], quad_swap<QUAD_XOR2>(x[i]));
  }
#pragma unroll
  for (int i = 0; i < 64; ++i) x[i] *= 0.0625f;
}

// x / s, equal to the IEEE fp32 quotient wherever that quotient can decide a
// code.  r is the correctly rounded 1 / s and s lies in [2^-30, 2^30]; the
// residual x - y s of y = x r is exact by FMA and one step y + r (x - y s)
// corrects it.  Quotients below 2^-20 in magnitude may differ in their last
// bits but keep the sign of x (every code rounds them to a signed zero),
// and y is held within +-2^80 so that huge quotients stay finite with the
// right sign (every code saturates there).  Checked against IEEE division
// for every bf16 x with every fp16 and UE4M3 scale, and for random fp32 x
// and per-tensor scales.
__device__ __forceinline__ float div_scale(float x, float s, float r) {
  const float y = __builtin_amdgcn_fmed3f(x * r, -0x1p80f, 0x1p80f);
  const float e = __builtin_fmaf(-y, s, x);
  return __builtin_copysignf(__builtin_fmaf(e, r, y), x);
}

// Two values -> two E4M3 codes in bytes 2 HI, 2 HI + 1 of `w` (RNE, saturating
// at +-448, sign kept).  v_cvt_pk_fp8_f32 rounds to nearest even over the
// whole grid but turns values past the 464 midpoint into NaN, so clamp first.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(uint32_t w, float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)w, HI);
}

// Two values -> two E2M1 codes in byte `sel` of `w`, a in the low nibble
// (RNE with ties to even, saturating at +-6, sign kept; checked against the
// format rule on every midpoint and a dense sweep of fp32 values).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t w, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, SEL);
}

// Round to nearest even and clamp to [-127, 127]; the low byte of the
// result is the two's-complement int8 code.  Adding 1.5 * 2^23 rounds a
// value below 2^22 in magnitude to an integer in the low mantissa bits.
__device__ __forceinline__ uint32_t i8_bits(float v) {
  v = __builtin_amdgcn_fmed3f(v, -127.0f, 127.0f);
  return __float_as_uint(v + 12582912.0f);
}

// Max of |x| over N elements.
template <int N>
__device__ __forceinline__ float abs_max(const float* x) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) a = fmaxf(a, fabsf(x[i]));
  return a;
}

// Codes of one lane's E values as little-endian packed words (element 0 in
// the lowest bits), BITS per code.
template <int C, int E, int BITS = codec_bits(C)>
struct Codes {
  uint32_t w[E * BITS / 32];
};

// Scale, reciprocal and stored scale bits of one group from its abs max.
template <int C>
__device__ __forceinline__ void group_scale(float amax, float& s, float& r, uint32_t& sbits) {
  if constexpr (C == C_I8G64 || C == C_E4ROW) {
    sbits = f16_scale_bits(__fdiv_rn(amax, C == C_I8G64 ? 127.0f : 448.0f));
    s = f16_bits_to_f32(sbits);
  } else if constexpr (C == C_E2G16) {
    sbits = e4m3_code(__fdiv_rn(amax, 6.0f));  // amax >= 0: the sign bit stays 0
    s = e4m3_value(sbits);
  } else {  // C_E4MX, C_E2MX: OCP MX shared exponent floor(log2 amax) - emax, biased by 127
    constexpr int EMAX = C == C_E4MX ? 8 : 2;  // largest exponent of E4M3, E2M1
    const int e = __builtin_amdgcn_frexp_expf(amax) - 1;
    int b = e - EMAX + 127;
    b = b < 0 ? 0 : (b > 254 ? 254 : b);
    sbits = amax > 0.0f ? (uint32_t)b : 0u;
    s = 1.0f;  // unused: the codes divide by 2^(sbits - 127) exactly with ldexp
  }
  r = s > 0.0f ? __fdiv_rn(1.0f, s) : 0.0f;
}

// Encode N consecutive values of one group (N a multiple of 8) into words
// starting at element `base` of the lane's run.
template <int C, int N, int E>
__device__ __forceinline__ void encode_group(const float* x, float s, float r, uint32_t sbits, Codes<C, E>& out,
                                             int base) {
  if constexpr (C == C_I8G64) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const uint32_t b0 = i8_bits(div_scale(x[i], s, r)), b1 = i8_bits(div_scale(x[i + 1], s, r));
      const uint32_t b2 = i8_bits(div_scale(x[i + 2], s, r)), b3 = i8_bits(div_scale(x[i + 3], s, r));
      const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);   // [b0.0, b1.0, 0, 0]
      const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x04000c0cu);   // [0, 0, b2.0, b3.0]
      out.w[(base + i) / 4] = s > 0.0f ? (lo | hi) : 0u;
    }
  } else if constexpr (C == C_E4ROW || C == C_E4MX) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = C == C_E4MX ? ldexpf(x[i + j], 127 - (int)sbits) : div_scale(x[i + j], s, r);
      uint32_t w = e4m3_pair<false>(0u, v[0], v[1]);
      w = e4m3_pair<true>(w, v[2], v[3]);
      out.w[(base + i) / 4] = (C == C_E4ROW && !(s > 0.0f)) ? 0u : w;
    }
  } else {  // C_E2G16, C_E2MX
#pragma unroll
    for (int i = 0; i < N; i += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = C == C_E2MX ? ldexpf(x[i + j], 127 - (int)sbits) : div_scale(x[i + j], s, r);
      uint32_t w = e2m1_pair<0>(0u, v[0], v[1]);
      w = e2m1_pair<1>(w, v[2], v[3]);
      w = e2m1_pair<2>(w, v[4], v[5]);
      w = e2m1_pair<3>(w, v[6], v[7]);
      out.w[(base + i) / 8] = (C == C_E2MX || s > 0.0f) ? w : 0u;
    }
  }
}

// ---------------------------------------------------------------- stores

// K codes at their tiled positions: element (t, d), kk = d/32, g = (d%32)/8,
// e = d%8: byte i*1024 + (g*16 + t)*16 + j*b/8 with i = kk/(16/b),
// j = (kk%(16/b))*8 + e.  Lane q holds d in [q E, (q + 1) E).
template <int BITS, int D>
__device__ __forceinline__ void store_k_codes(uint8_t* codes, const uint32_t* w, int q, int t) {
  constexpr int E = D / 4;
  if constexpr (BITS == 8) {
    if constexpr (E == 64) {  // k-steps 2q, 2q+1: one whole 16-byte chunk per g
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<uint4*>(codes + q * 1024 + (g * 16 + t) * 16) =
            make_uint4(w[2 * g], w[2 * g + 1], w[8 + 2 * g], w[9 + 2 * g]);
    } else {  // E == 32: k-step q, the half (q % 2) of chunk q / 2
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<uint2*>(codes + (q >> 1) * 1024 + (g * 16 + t) * 16 + (q & 1) * 8) =
            make_uint2(w[2 * g], w[2 * g + 1]);
    }
  } else if constexpr (BITS == 4) {  // D == 256: k-steps 2q, 2q+1 are the half (q % 2) of chunk q / 2
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<uint2*>(codes + (q >> 1) * 1024 + (g * 16 + t) * 16 + (q & 1) * 8) = make_uint2(w[g], w[4 + g]);
  } else {  // 16-bit: one k-step per chunk
#pragma unroll
    for (int kl = 0; kl < E / 32; ++kl)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<uint4*>(codes + (q * (E / 32) + kl) * 1024 + (g * 16 + t) * 16) =
            make_uint4(w[16 * kl + 4 * g], w[16 * kl + 4 * g + 1], w[16 * kl + 4 * g + 2], w[16 * kl + 4 * g + 3]);
  }
}

// Two-level NVFP4: the (rotated) row is divided by the per-tensor scale g
// before its groups are scaled, in IEEE fp32 (div_scale's quotient is the
// IEEE one wherever it can reach a code or a group maximum that is not
// flushed to a zero scale); g = 1 leaves the row unchanged.
template <int N>
__device__ __forceinline__ void divide_by_tensor_scale(float (&x)[N], float g) {
  if (g == 1.0f) return;  // uniform
  const float r = __fdiv_rn(1.0f, g);
  const bool fast = g >= 0x1p-30f && g <= 0x1p30f;
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = fast ? div_scale(x[i], g, r) : __fdiv_rn(x[i], g);
}

// ---------------------------------------------------------------- one plane

template <int C, int D, bool ROT, int PLANE>
__device__ __forceinline__ void encode_plane(float (&x)[D / 4], int q, uint8_t* codes, uint8_t* scales, int t,
                                             float tensor_scale) {
  constexpr int E = D / 4;
  constexpr int BITS = codec_bits(C);
  if constexpr (ROT) {
    static_assert(D == 256, "the rotation is 256-point");
    fwht256_quad(x, q);
  }
  if constexpr (C == C_E2G16) divide_by_tensor_scale(x, tensor_scale);
  Codes<C, E> out;
  if constexpr (C == C_F16) {
#pragma unroll
    for (int i = 0; i < E; i += 2) out.w[i / 2] = f16_bits(x[i]) | (f16_bits(x[i + 1]) << 16);
  } else if constexpr (C == C_E4TEN) {
    const float s = tensor_scale, r = __fdiv_rn(1.0f, s);
    const bool fast = s >= 0x1p-30f && s <= 0x1p30f;  // uniform
#pragma unroll
    for (int i = 0; i < E; i += 4) {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = fast ? div_scale(x[i + j], s, r) : __fdiv_rn(x[i + j], s);
      const uint32_t w = e4m3_pair<false>(0u, v[0], v[1]);
      out.w[i / 4] = e4m3_pair<true>(w, v[2], v[3]);
    }
  } else {
    constexpr int GS = codec_group(C) < 0 ? D : codec_group(C);
    constexpr int G = D / GS;
    if constexpr (GS > E) {  // one group spans the quad: the row-wide FP8 scale
      float amax = abs_max<E>(x);
      amax = fmaxf(amax, quad_swap<QUAD_XOR1>(amax));
      amax = fmaxf(amax, quad_swap<QUAD_XOR2>(amax));
      float s, r;
      uint32_t sbits;
      group_scale<C>(amax, s, r, sbits);
      encode_group<C, E, E>(x, s, r, sbits, out, 0);
      if (q == 0) *reinterpret_cast<uint16_t*>(scales + t * G * 2) = (uint16_t)sbits;
    } else {
      constexpr int GPL = E / GS;  // groups per lane
      uint32_t sb[GPL];
#pragma unroll
      for (int gl = 0; gl < GPL; ++gl) {
        float s, r;
        group_scale<C>(abs_max<GS>(x + gl * GS), s, r, sb[gl]);
        encode_group<C, GS, E>(x + gl * GS, s, r, sb[gl], out, gl * GS);
      }
      const int grp0 = q * GPL;
      if constexpr (scale_bytes(C) == 2) {  // INT8-G64: one group per lane (D = 256)
        static_assert(GPL == 1, "");
        *reinterpret_cast<uint16_t*>(scales + (t * G + grp0) * 2) = (uint16_t)sb[0];
      } else if constexpr (GPL == 4) {
        *reinterpret_cast<uint32_t*>(scales + t * G + grp0) = sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
      } else if constexpr (GPL == 2) {
        *reinterpret_cast<uint16_t*>(scales + t * G + grp0) = (uint16_t)(sb[0] | (sb[1] << 8));
      } else {
        scales[t * G + grp0] = (uint8_t)sb[0];
      }
    }
  }
  static_assert(PLANE == 0, "V rows are encoded by v_row_group");
  store_k_codes<BITS, D>(codes, out.w, q, t);
}

// ---------------------------------------------------------------- V waves

// Fixed-order FWHT-256 scaled by 2^-4 of one row held by 16 lanes, lane j
// holding elements 16 j .. 16 j + 15: stages h = 1 .. 8 inside the lane,
// then h = 16, 32, 64, 128 between lanes j and j ^ (h / 16), the lower lane
// keeping the sum and the upper one the difference.
__device__ __forceinline__ void fwht256_row16(float (&x)[16], int j) {
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
#define KVQ_CROSS(M)                                                                            \
  {                                                                                             \
    const float sg = (j & M) ? -1.0f : 1.0f;                                                    \
    _Pragma("unroll") for (int i = 0; i < 16; ++i) x[i] = __builtin_fmaf(sg, x[i], lane_xor<M>(x[i])); \
  }
  KVQ_CROSS(1) KVQ_CROSS(2) KVQ_CROSS(4) KVQ_CROSS(8)
#undef KVQ_CROSS
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] *= 0.0625f;
}

// Codes of element i of the lane for all 4 tokens: one 32-bit word per i
// holding token e in byte e (8-bit codes), two words per i holding tokens
// (0, 1) and (2, 3) (16-bit codes), or, for 4-bit codes, one word per
// m < F / 2 holding elements 2m and 2m + 1: bytes 0, 1 hold element 2m of
// tokens (0, 1) and (2, 3), bytes 2, 3 element 2m + 1, the earlier token of
// each pair in the low nibble (the tile's byte order).
template <int C, int F>
struct VWords {
  static constexpr int N = codec_bits(C) == 16 ? 2 * F : codec_bits(C) == 8 ? F : F / 2;
  uint32_t w[N];
};

// Store tokens first .. first + n - 1 (0 <= first, first + n <= 4) of a
// group of 4 tokens packed TB bytes each in W (token e in bytes TB e ..
// TB e + TB - 1) at p, which holds the group's 4 TB bytes.
template <int TB>
__device__ __forceinline__ void store_tokens(uint8_t* p, uint64_t W, int first, int n) {
  const uint64_t v = W >> (8 * TB * first);
  uint8_t* q = p + TB * first;
  const int bytes = TB * n;
  if (bytes == 1) {
    q[0] = (uint8_t)v;
  } else if (bytes == 2) {
    *reinterpret_cast<uint16_t*>(q) = (uint16_t)v;
  } else if (bytes == 3) {  // first is 0 or 1 (TB == 1)
    if (first == 0) {
      *reinterpret_cast<uint16_t*>(q) = (uint16_t)v;
      q[2] = (uint8_t)(v >> 16);
    } else {
      q[0] = (uint8_t)v;
      *reinterpret_cast<uint16_t*>(q + 1) = (uint16_t)(v >> 8);
    }
  } else if (bytes == 4) {
    *reinterpret_cast<uint32_t*>(q) = (uint32_t)v;
  } else {  // 6 bytes: tokens 0 .. 2 or 1 .. 3 of 2-byte tokens
    if (first == 0) {
      *reinterpret_cast<uint32_t*>(q) = (uint32_t)v;
      *reinterpret_cast<uint16_t*>(q + 4) = (uint16_t)(v >> 32);
    } else {
      *reinterpret_cast<uint16_t*>(q) = (uint16_t)v;
      *reinterpret_cast<uint32_t*>(q + 2) = (uint32_t)(v >> 16);
    }
  }
}

// Store the 4-bit V codes of token e of a row's 4 (codes in the tile byte
// order of VWords, lane j holding n-tile j) at slab position te of slab gv
// of the token block at `codes`, leaving the other tokens' nibbles intact.
// The quad of n-tiles 4q .. 4q + 3 covers 8 bytes of every tile row (row n
// of chunk q / 2, bytes 8 (q % 2) .. + 7); the nibbles are first gathered
// across the quad so that lane k holds those 8 bytes' worth of rows
// n = k + 4m, and each lane then does 64-bit and/or on 4 distinct words.
__device__ __forceinline__ void store_token_nibbles(uint8_t* codes, const uint32_t (&w)[8], int e, int gv, int te,
                                                    int j) {
  const int k = j & 3, q = j >> 2;
  // this token's nibble of column n: word n / 2, bits 16 (n % 2) + se
  const int se = 8 * (e >> 1) + 4 * (e & 1);
  uint32_t x[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) x[m] = (w[m] >> se) & 0x000F000Fu;
  // E[r] (16 bits, nibble i = column r + 4 i): V0 = (E[0], E[1]), V1 = (E[2], E[3])
  const uint32_t V0 = x[0] | (x[2] << 4) | (x[4] << 8) | (x[6] << 12);
  const uint32_t V1 = x[1] | (x[3] << 4) | (x[5] << 8) | (x[7] << 12);
  // transpose E across the quad: lane k ends with E of every n-tile for r = k
  const bool b1 = (k & 2) != 0, b0 = (k & 1) != 0;
  const uint32_t A = b1 ? V1 : V0;                       // own E[rb], E[rb + 1], rb = 2 b1
  const uint32_t B = lane_xor_u32<2>(b1 ? V0 : V1);      // lane k ^ 2's
  const uint32_t lo = __builtin_amdgcn_perm(B, A, 0x05040100u), hi = __builtin_amdgcn_perm(B, A, 0x07060302u);
  const uint32_t keep = b0 ? hi : lo;                    // (E_k, E_{k^2}) for r = k
  const uint32_t R = lane_xor_u32<1>(b0 ? lo : hi);      // (E_{k^1}, E_{k^3}) for r = k
  const uint32_t X = b0 ? R : keep, Y = b0 ? keep : R;   // n-tiles (0, 2) and (1, 3), swapped when b1
  const uint32_t xy_lo = __builtin_amdgcn_perm(Y, X, 0x05040100u), xy_hi = __builtin_amdgcn_perm(Y, X, 0x07060302u);
  const uint32_t P = b1 ? xy_hi : xy_lo;                 // n-tiles 4q, 4q + 1 at bits 0, 16
  const uint32_t Q = b1 ? xy_lo : xy_hi;                 // n-tiles 4q + 2, 4q + 3
  const int st = 8 * (te >> 1) + 4 * (te & 1);           // the slot's nibble in its byte pair
  const uint64_t mask = 0x000F000F000F000Full << st;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint64_t v = ((uint64_t)((Q >> (4 * m)) & 0x000F000Fu) << 32) | ((P >> (4 * m)) & 0x000F000Fu);
    unsigned long long* wp = reinterpret_cast<unsigned long long*>(
        codes + (q >> 1) * 1024 + (gv * 16 + k + 4 * m) * 16 + (q & 1) * 8);
    atomicAnd(wp, ~mask);
    atomicOr(wp, v << st);
  }
}

// Encode and store the V rows of tokens t0 .. t0 + 3 of kv head `head`, held
// by this row of 16 lanes (lane j); tokens outside [tlo, thi) are left out.
// slot_of(token) gives a token's slot (negative: not stored); the input row
// of token t is v[(t * H_kv + head) * D ...].
template <int FMT, int D, typename SlotOf>
__device__ __forceinline__ void v_row_group(uint8_t* __restrict__ pool, const uint16_t* __restrict__ v,
                                            SlotOf slot_of, const Geometry& geo, float v_scale,
                                            int head, int j, int64_t t0, int64_t tlo, int64_t thi) {
  constexpr int C = v_codec(FMT);
  constexpr int F = D / 16;
  constexpr int BITS = codec_bits(C);
  int slot[4];
  bool ok[4];
  uint32_t raw[4][F / 2];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t tok = t0 + e;
    const bool in = tok >= tlo && tok < thi;
    slot[e] = in ? slot_of(tok) : -1;
    ok[e] = slot[e] >= 0;
    if (in) {  // loaded whatever the slot says, so the two loads overlap
      const uint16_t* src = v + (tok * geo.H_kv + head) * D + j * F;
#pragma unroll
      for (int i = 0; i < F / 8; ++i) {
        const uint4 w = *reinterpret_cast<const uint4*>(src + 8 * i);
        raw[e][4 * i] = w.x; raw[e][4 * i + 1] = w.y; raw[e][4 * i + 2] = w.z; raw[e][4 * i + 3] = w.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < F / 2; ++i) raw[e][i] = 0u;
    }
  }

  // ---- codes, two tokens at a time (one scale per token for the lane's group)
  VWords<C, F> out;
  constexpr int GS = codec_group(C) <= 0 ? D : codec_group(C);  // no scales: indexes only
  uint32_t sb[4] = {0u, 0u, 0u, 0u};
  uint32_t keep = 0xFFFFFFFFu;  // byte e cleared where token e's group scale is 0
#pragma unroll
  for (int pr = 0; pr < 2; ++pr) {
    float x[2][F];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < F / 2; ++i) {
        x[h2][2 * i] = bf16_to_f32(raw[2 * pr + h2][i] & 0xFFFFu);
        x[h2][2 * i + 1] = bf16_to_f32(raw[2 * pr + h2][i] >> 16);
      }
    if constexpr (v_rotated(FMT)) {
      static_assert(D == 256, "the rotation is 256-point");
      fwht256_row16(x[0], j);
      fwht256_row16(x[1], j);
    }
    if constexpr (C == C_E2G16) {
      divide_by_tensor_scale(x[0], v_scale);
      divide_by_tensor_scale(x[1], v_scale);
    }
    if constexpr (C == C_F16) {
#pragma unroll
      for (int i = 0; i < F; ++i) out.w[2 * i + pr] = f16_bits(x[0][i]) | (f16_bits(x[1][i]) << 16);
    } else {
      float s[2], r[2];
      bool fast = true;
      if constexpr (C == C_E4TEN) {
        const float rr = __fdiv_rn(1.0f, v_scale);
        fast = v_scale >= 0x1p-30f && v_scale <= 0x1p30f;  // uniform
        s[0] = s[1] = v_scale;
        r[0] = r[1] = rr;
      } else {
        static_assert(GS >= F, "a group spans whole lanes");
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const float amax = max_over_lanes<GS / F>(abs_max<F>(x[h2]));
          group_scale<C>(amax, s[h2], r[h2], sb[2 * pr + h2]);
          if constexpr (!mx_scaled(C))
            if (!(s[h2] > 0.0f))
              keep &= BITS == 4 ? ~(0x000F000Fu << (8 * pr + 4 * h2)) : ~(0xFFu << (8 * (2 * pr + h2)));
        }
      }
      auto quot = [&](int h2, float xv) -> float {
        if constexpr (mx_scaled(C)) return ldexpf(xv, 127 - (int)sb[2 * pr + h2]);
        else return fast ? div_scale(xv, s[h2], r[h2]) : __fdiv_rn(xv, s[h2]);
      };
      if constexpr (BITS == 8) {
#pragma unroll
        for (int i = 0; i < F; ++i) {
          if constexpr (C == C_I8G64) {
            const uint32_t b0 = i8_bits(quot(0, x[0][i])), b1 = i8_bits(quot(1, x[1][i]));
            const uint32_t w = __builtin_amdgcn_perm(b1, b0, pr ? 0x04000c0cu : 0x0c0c0400u);
            out.w[i] = pr ? (out.w[i] | w) : w;
          } else {
            out.w[i] = pr ? e4m3_pair<true>(out.w[i], quot(0, x[0][i]), quot(1, x[1][i]))
                          : e4m3_pair<false>(0u, quot(0, x[0][i]), quot(1, x[1][i]));
          }
        }
      } else {  // 4-bit: one element of tokens 2 pr and 2 pr + 1 per byte
#pragma unroll
        for (int m = 0; m < F / 2; ++m) {
          uint32_t w = pr ? out.w[m] : 0u;
          if (pr == 0) {
            w = e2m1_pair<0>(w, quot(0, x[0][2 * m]), quot(1, x[1][2 * m]));
            w = e2m1_pair<2>(w, quot(0, x[0][2 * m + 1]), quot(1, x[1][2 * m + 1]));
          } else {
            w = e2m1_pair<1>(w, quot(0, x[0][2 * m]), quot(1, x[1][2 * m]));
            w = e2m1_pair<3>(w, quot(0, x[0][2 * m + 1]), quot(1, x[1][2 * m + 1]));
          }
          out.w[m] = w;
        }
      }
    }
  }
  if constexpr (C != C_F16) {
#pragma unroll
    for (int i = 0; i < VWords<C, F>::N; ++i) out.w[i] &= keep;
  }

  // ---- stores.  Element i of lane j: d = j F + i, n-tile jt = d / 16, n = d % 16.
  const int jt = (j * F) >> 4, n0 = (j * F) & 15;
  const int grp = (j * F) / GS;
  const bool lead = ((j * F) % GS) == 0;  // the lane that stores its group's scales
  constexpr int G = D / GS;
  const bool slab = ok[0] && ok[1] && ok[2] && ok[3] && (slot[0] & 3) == 0 && slot[1] == slot[0] + 1 &&
                    slot[2] == slot[0] + 2 && slot[3] == slot[0] + 3;
  if (slab) {
    const int64_t page = slot[0] / geo.P;
    const int off = slot[0] - (int)(page * geo.P);
    const int blk = off >> 4, gv = (off & 15) >> 2;
    uint8_t* hb = pool + page * geo.page_bytes + (int64_t)head * geo.head_bytes;
    uint8_t* codes = hb + geo.off_vc + (int64_t)blk * geo.vcode_blk;
    uint8_t* scales = hb + geo.off_vs + (int64_t)blk * geo.vscale_blk;
    if constexpr (D == 256 && BITS == 8) {
      // the 16-byte tile chunk of n-tiles 4a .. 4a + 3 (lanes 4a + c) and one
      // n: transpose each 4 x 4 block of words across the quad so that lane
      // c holds the chunk of n = 4 m + c
#pragma unroll
      for (int m = 0; m < F / 4; ++m) {
        uint32_t W[4] = {out.w[4 * m], out.w[4 * m + 1], out.w[4 * m + 2], out.w[4 * m + 3]};
        quad_transpose(W, j & 3);
        const int n = 4 * m + (j & 3);
        *reinterpret_cast<uint4*>(codes + (jt >> 2) * 1024 + (gv * 16 + n) * 16) = make_uint4(W[0], W[1], W[2], W[3]);
      }
    } else if constexpr (D == 256 && BITS == 4) {
      // the 16-byte tile rows n of chunk jt / 8 hold n-tiles 8c .. 8c + 7
      // (lanes 8c + k), 2 bytes each: transpose the 8 x 8 words across the
      // group so that lane k holds columns 2k and 2k + 1 of all 8 n-tiles,
      // then the low halves form row n = 2k and the high halves row 2k + 1
      const int k = j & 7;
      uint32_t W[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) W[m] = out.w[m];
      oct_transpose(W, k);
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo[i] = __builtin_amdgcn_perm(W[2 * i + 1], W[2 * i], 0x05040100u);
        hi[i] = __builtin_amdgcn_perm(W[2 * i + 1], W[2 * i], 0x07060302u);
      }
      uint8_t* dst = codes + (jt >> 3) * 1024 + (gv * 16 + 2 * k) * 16;
      *reinterpret_cast<uint4*>(dst) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    } else if constexpr (D == 256) {
      // 16-bit: the chunk of n-tiles 2b, 2b + 1 (lanes 2b + p) and one n;
      // lane p of a pair assembles n = 2 q + p
      const int p = j & 1;
#pragma unroll
      for (int q2 = 0; q2 < F / 2; ++q2) {
        const uint32_t s0 = p ? out.w[4 * q2] : out.w[4 * q2 + 2];
        const uint32_t s1 = p ? out.w[4 * q2 + 1] : out.w[4 * q2 + 3];
        const uint32_t r0 = lane_xor_u32<1>(s0), r1 = lane_xor_u32<1>(s1);
        const uint4 c4 = p ? make_uint4(r0, r1, out.w[4 * q2 + 2], out.w[4 * q2 + 3])
                           : make_uint4(out.w[4 * q2], out.w[4 * q2 + 1], r0, r1);
        *reinterpret_cast<uint4*>(codes + (jt >> 1) * 1024 + (gv * 16 + 2 * q2 + p) * 16) = c4;
      }
    } else if constexpr (BITS == 8) {
#pragma unroll
      for (int i = 0; i < F; ++i)
        *reinterpret_cast<uint32_t*>(codes + (jt >> 2) * 1024 + (gv * 16 + n0 + i) * 16 + (jt & 3) * 4) = out.w[i];
    } else {
#pragma unroll
      for (int i = 0; i < F; ++i)
        *reinterpret_cast<uint2*>(codes + (jt >> 1) * 1024 + (gv * 16 + n0 + i) * 16 + (jt & 1) * 8) =
            make_uint2(out.w[2 * i], out.w[2 * i + 1]);
    }
    if constexpr (scale_bytes(C) > 0) {
      if (lead) {
        const int tb = off & 15;  // block-local slot of token 0
        if constexpr (BITS == 4) {  // 4-bit V scales of tokens 4 gv + e at gv*4G + grp*4 + e
          *reinterpret_cast<uint32_t*>(scales + gv * 4 * G + grp * 4) = sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
        } else if constexpr (scale_bytes(C) == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) *reinterpret_cast<uint16_t*>(scales + ((tb + e) * G + grp) * 2) = (uint16_t)sb[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) scales[(tb + e) * G + grp] = (uint8_t)sb[e];
        }
      }
    }
  } else if (BITS != 4 && ok[0] && ok[1] && ok[2] && ok[3] && slot[1] == slot[0] + 1 &&
             slot[2] == slot[0] + 2 && slot[3] == slot[0] + 3) {
    // consecutive slots s0 .. s0 + 3 with a = s0 % 4 != 0: tokens 0 .. 3 - a
    // go to positions a .. 3 of slab s0 - a, tokens 4 - a .. 3 to positions
    // 0 .. a - 1 of the next slab (4-bit codes share bytes between tokens
    // and take the per-token path below)
    const int a = slot[0] & 3;
    uint8_t* cw[2];
    int gvv[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int sl = slot[0] - a + 4 * h2;  // first slot of each slab
      const int64_t page = sl / geo.P;
      const int off = sl - (int)(page * geo.P);
      gvv[h2] = (off & 15) >> 2;
      cw[h2] = pool + page * geo.page_bytes + (int64_t)head * geo.head_bytes + geo.off_vc +
               (int64_t)(off >> 4) * geo.vcode_blk;
    }
#pragma unroll
    for (int i = 0; i < F; ++i) {
      int o[2];
      uint64_t W;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        o[h2] = BITS == 8 ? (jt >> 2) * 1024 + (gvv[h2] * 16 + n0 + i) * 16 + (jt & 3) * 4
                          : (jt >> 1) * 1024 + (gvv[h2] * 16 + n0 + i) * 16 + (jt & 1) * 8;
      if constexpr (BITS == 16) W = (uint64_t)out.w[2 * i] | ((uint64_t)out.w[2 * i + 1] << 32);
      else W = out.w[i];
      constexpr int TB = BITS == 16 ? 2 : 1;
      store_tokens<TB>(cw[0] + o[0], W << (8 * TB * a), a, 4 - a);
      store_tokens<TB>(cw[1] + o[1], W >> (8 * TB * (4 - a)), 0, a);
    }
    if constexpr (scale_bytes(C) > 0) {
      if (lead) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int sl = slot[e];
          const int64_t page = sl / geo.P;
          const int off = sl - (int)(page * geo.P);
          const int t = off & 15;
          uint8_t* scales = pool + page * geo.page_bytes + (int64_t)head * geo.head_bytes + geo.off_vs +
                            (int64_t)(off >> 4) * geo.vscale_blk;
          if constexpr (BITS == 4) scales[(t >> 2) * 4 * G + grp * 4 + (t & 3)] = (uint8_t)sb[e];
          else if constexpr (scale_bytes(C) == 2) *reinterpret_cast<uint16_t*>(scales + (t * G + grp) * 2) = (uint16_t)sb[e];
          else scales[t * G + grp] = (uint8_t)sb[e];
        }
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!ok[e]) continue;
      const int64_t page = slot[e] / geo.P;
      const int off = slot[e] - (int)(page * geo.P);
      const int blk = off >> 4, t = off & 15, gv = t >> 2, te = t & 3;
      uint8_t* hb = pool + page * geo.page_bytes + (int64_t)head * geo.head_bytes;
      uint8_t* codes = hb + geo.off_vc + (int64_t)blk * geo.vcode_blk;
      uint8_t* scales = hb + geo.off_vs + (int64_t)blk * geo.vscale_blk;
      if constexpr (BITS == 8) {
#pragma unroll
        for (int i = 0; i < F; ++i)
          codes[(jt >> 2) * 1024 + (gv * 16 + n0 + i) * 16 + (jt & 3) * 4 + te] = (uint8_t)(out.w[i] >> (8 * e));
      } else if constexpr (BITS == 16) {
#pragma unroll
        for (int i = 0; i < F; ++i)
          *reinterpret_cast<uint16_t*>(codes + (jt >> 1) * 1024 + (gv * 16 + n0 + i) * 16 + (jt & 1) * 8 + 2 * te) =
              (uint16_t)(out.w[2 * i + (e >> 1)] >> (16 * (e & 1)));
      } else {
        // 4-bit: this token's nibble of each column shares its byte with
        // the other token of its pair (written by this call or another), so
        // the nibbles are set with atomic and/or, which leave the partner's
        // bits alone whoever writes them and in whatever order
        static_assert(F == 16, "one n-tile per lane");
        store_token_nibbles(codes, out.w, e, gv, te, j);
      }
      if constexpr (scale_bytes(C) > 0) {
        if (lead) {
          if constexpr (BITS == 4) scales[gv * 4 * G + grp * 4 + te] = (uint8_t)sb[e];
          else if constexpr (scale_bytes(C) == 2) *reinterpret_cast<uint16_t*>(scales + (t * G + grp) * 2) = (uint16_t)sb[e];
          else scales[t * G + grp] = (uint8_t)sb[e];
        }
      }
    }
  }
}

// Encode the K row of one token for kv head `head` and store it at `slot`:
// the 4 lanes of a quad (lane q) each hold raw bf16 elements [q D/4, (q+1) D/4).
template <int FMT, int D>
__device__ __forceinline__ void encode_k_row(uint8_t* __restrict__ pool, const uint32_t (&raw)[D / 8], int slot,
                                             const Geometry& geo, int head, float k_scale, int q) {
  constexpr int E = D / 4;
  const int64_t page = slot / geo.P;
  const int off = slot - (int)(page * geo.P);
  const int blk = off >> 4, t = off & 15;
  uint8_t* head_base = pool + page * geo.page_bytes + (int64_t)head * geo.head_bytes;
  uint8_t* codes = head_base + geo.off_kc + (int64_t)blk * geo.kcode_blk;
  uint8_t* scales = head_base + geo.off_ks + (int64_t)blk * geo.kscale_blk;
  constexpr int KC = k_codec(FMT);
  if constexpr (KC == C_BF16) {
    store_k_codes<16, D>(codes, raw, q, t);  // K of BF16 is stored bit for bit
  } else {
    float x[E];
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
      x[2 * i] = bf16_to_f32(raw[i] & 0xFFFFu);
      x[2 * i + 1] = bf16_to_f32(raw[i] >> 16);
    }
    encode_plane<KC, D, k_rotated(FMT), 0>(x, q, codes, scales, t, k_scale);
  }
}

// Load the raw bf16 K elements [q D/4, (q+1) D/4) of one input row.
template <int D>
__device__ __forceinline__ void load_k_row(uint32_t (&raw)[D / 8], const uint16_t* src) {
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    const uint4 w = *reinterpret_cast<const uint4*>(src + 8 * i);
    raw[4 * i] = w.x; raw[4 * i + 1] = w.y; raw[4 * i + 2] = w.z; raw[4 * i + 3] = w.w;
  }
}


// ---------------------------------------------------------- single tokens
// One token's K or V row held by a whole wave, for appends of a few tokens
// (a decode step adds one per sequence), where the rows above leave most
// lanes idle and give each busy lane a long serial chain.  N = D / 64
// elements per lane:
//
//   K: lane l holds d = N l .. N l + N - 1 (the row in order), so its codes
//      are N consecutive values of one K tile row;
//   V: lane l = 16 Q + n holds d = 16 (N Q + k) + n, k < N: column n of
//      n-tiles N Q .. N Q + N - 1, so its codes sit in one V tile row.
//
// The rotation runs the stages h = 1, 2, ..., 128 in that order, each
// pairing the same two elements with one rounding, and every other step is
// elementwise or an exact maximum, so the stored bytes are those of the
// row encoders above.  Every lane of the wave must take part.

// Max over the L lanes (L a power of two <= 64) whose index differs only in
// its low log2 L bits.
template <int L>
__device__ __forceinline__ float max_over_lanes_wave(float a) {
  a = max_over_lanes<(L < 16 ? L : 16)>(a);
  if constexpr (L >= 32) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
    a = fmaxf(__uint_as_float((uint32_t)s[0]), __uint_as_float((uint32_t)s[1]));
  }
  if constexpr (L >= 64) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
    a = fmaxf(__uint_as_float((uint32_t)s[0]), __uint_as_float((uint32_t)s[1]));
  }
  return a;
}

// Raw bf16 elements of one token row in the wave's K or V order, two per word.
template <int D>
struct TokenRow {
  uint32_t w[D / 128];
};

template <int D>
__device__ __forceinline__ void load_k_token(TokenRow<D>& r, const uint16_t* row, int lane) {
  if constexpr (D == 256) {
    const uint2 w = *reinterpret_cast<const uint2*>(row + 4 * lane);
    r.w[0] = w.x;
    r.w[1] = w.y;
  } else {
    static_assert(D == 128, "");
    r.w[0] = *reinterpret_cast<const uint32_t*>(row + 2 * lane);
  }
}

template <int D>
__device__ __forceinline__ void load_v_token(TokenRow<D>& r, const uint16_t* row, int lane) {
  constexpr int N = D / 64;
  const uint16_t* p = row + 16 * N * (lane >> 4) + (lane & 15);
#pragma unroll
  for (int i = 0; i < N / 2; ++i) r.w[i] = (uint32_t)p[32 * i] | ((uint32_t)p[32 * i + 16] << 16);
}

template <int D>
__device__ __forceinline__ void unpack_token(const TokenRow<D>& r, float (&x)[D / 64]) {
#pragma unroll
  for (int i = 0; i < D / 128; ++i) {
    x[2 * i] = bf16_to_f32(r.w[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_to_f32(r.w[i] >> 16);
  }
}

// Quotient of x by its group scale, as the row encoders take it.
template <int C>
__device__ __forceinline__ float token_quot(float x, float s, float r, uint32_t sbits, bool fast) {
  if constexpr (mx_scaled(C)) return ldexpf(x, 127 - (int)sbits);
  else if constexpr (C == C_E4TEN) return fast ? div_scale(x, s, r) : __fdiv_rn(x, s);
  else return div_scale(x, s, r);
}

// The code of one quotient in the low BITS bits.
template <int C>
__device__ __forceinline__ uint32_t token_code(float q) {
  if constexpr (C == C_I8G64) return i8_bits(q) & 0xFFu;
  else if constexpr (codec_bits(C) == 8) return e4m3_pair<false>(0u, q, 0.0f) & 0xFFu;
  else return e2m1_pair<0>(0u, q, 0.0f) & 0xFu;
}

// Encode one token's K row (TokenRow in K order) and store it at `slot`.
template <int FMT, int D>
__device__ __forceinline__ void encode_k_token(uint8_t* __restrict__ pool, const TokenRow<D>& raw, int slot,
                                               const Geometry& geo, int head, float k_scale, int lane) {
  constexpr int N = D / 64;
  constexpr int C = k_codec(FMT);
  constexpr int BITS = codec_bits(C);
  const int64_t page = slot / geo.P;
  const int off = slot - (int)(page * geo.P);
  const int blk = off >> 4, t = off & 15;
  uint8_t* head_base = pool + page * geo.page_bytes + (int64_t)head * geo.head_bytes;
  uint8_t* codes = head_base + geo.off_kc + (int64_t)blk * geo.kcode_blk;
  uint8_t* scales = head_base + geo.off_ks + (int64_t)blk * geo.kscale_blk;
  const int d0 = N * lane;
  uint8_t* dst = codes + k_code_byte(BITS, t, d0);
  if constexpr (C == C_BF16) {  // K of BF16 is stored bit for bit
    if constexpr (N == 4) *reinterpret_cast<uint2*>(dst) = make_uint2(raw.w[0], raw.w[1]);
    else *reinterpret_cast<uint32_t*>(dst) = raw.w[0];
    return;
  } else {
    float x[N];
    unpack_token<D>(raw, x);
    if constexpr (k_rotated(FMT)) {
      static_assert(D == 256, "the rotation is 256-point");
      // h = 1, 2 inside the lane, h = 4 .. 128 across lanes 1 .. 32 apart
#pragma unroll
      for (int h = 1; h < N; h <<= 1)
#pragma unroll
        for (int i = 0; i < N; ++i)
          if ((i & h) == 0) {
            const float a = x[i], b = x[i + h];
            x[i] = a + b;
            x[i + h] = a - b;
          }
#pragma unroll
      for (int i = 0; i < N; ++i) {
        x[i] = xlane_butterfly<1>(x[i], lane);
        x[i] = xlane_butterfly<2>(x[i], lane);
        x[i] = xlane_butterfly<4>(x[i], lane);
        x[i] = xlane_butterfly<8>(x[i], lane);
        x[i] = xlane_butterfly<16>(x[i], lane);
        x[i] = xlane_butterfly<32>(x[i], lane);
        x[i] *= 0.0625f;
      }
    }
    if constexpr (C == C_E2G16) divide_by_tensor_scale(x, k_scale);
    float s = k_scale, r = 0.0f;
    uint32_t sbits = 0u;
    bool fast = true, zero = false;
    if constexpr (C == C_E4TEN) {
      r = __fdiv_rn(1.0f, s);
      fast = s >= 0x1p-30f && s <= 0x1p30f;  // uniform
    } else {
      constexpr int GS = codec_group(C) < 0 ? D : codec_group(C);
      group_scale<C>(max_over_lanes_wave<GS / N>(abs_max<N>(x)), s, r, sbits);
      zero = !mx_scaled(C) && !(s > 0.0f);
      if ((d0 % GS) == 0) {  // the group's first lane stores its scale
        constexpr int G = D / GS;
        const int grp = d0 / GS;
        if constexpr (scale_bytes(C) == 2) *reinterpret_cast<uint16_t*>(scales + (t * G + grp) * 2) = (uint16_t)sbits;
        else scales[t * G + grp] = (uint8_t)sbits;
      }
    }
    uint32_t w = 0u;
#pragma unroll
    for (int i = 0; i < N; ++i) w |= token_code<C>(token_quot<C>(x[i], s, r, sbits, fast)) << (BITS * i);
    if (zero) w = 0u;
    if constexpr (BITS * N == 32) *reinterpret_cast<uint32_t*>(dst) = w;
    else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w;
  }
}

// Encode one token's V row (TokenRow in V order) and store it at `slot`.
// 8- and 16-bit codes share their tile words with the slab's other tokens
// and are written byte- or halfword-wise; 4-bit codes share bytes with the
// other token of their pair and are set with atomic and/or.
template <int FMT, int D>
__device__ __forceinline__ void encode_v_token(uint8_t* __restrict__ pool, const TokenRow<D>& raw, int slot,
                                               const Geometry& geo, int head, float v_scale, int lane) {
  constexpr int N = D / 64;
  constexpr int C = v_codec(FMT);
  constexpr int BITS = codec_bits(C);
  const int Q = lane >> 4, n = lane & 15;
  const int64_t page = slot / geo.P;
  const int off = slot - (int)(page * geo.P);
  const int blk = off >> 4, t = off & 15, gv = t >> 2, te = t & 3;
  uint8_t* head_base = pool + page * geo.page_bytes + (int64_t)head * geo.head_bytes;
  uint8_t* codes = head_base + geo.off_vc + (int64_t)blk * geo.vcode_blk;
  uint8_t* scales = head_base + geo.off_vs + (int64_t)blk * geo.vscale_blk;
  float x[N];
  unpack_token<D>(raw, x);
  if constexpr (v_rotated(FMT)) {
    static_assert(D == 256, "the rotation is 256-point");
    // h = 1 .. 8 across lanes 1 .. 8 apart, h = 16, 32 inside the lane,
    // h = 64, 128 across lanes 16, 32 apart
#pragma unroll
    for (int i = 0; i < N; ++i) {
      x[i] = xlane_butterfly<1>(x[i], lane);
      x[i] = xlane_butterfly<2>(x[i], lane);
      x[i] = xlane_butterfly<4>(x[i], lane);
      x[i] = xlane_butterfly<8>(x[i], lane);
    }
#pragma unroll
    for (int h = 1; h < N; h <<= 1)
#pragma unroll
      for (int i = 0; i < N; ++i)
        if ((i & h) == 0) {
          const float a = x[i], b = x[i + h];
          x[i] = a + b;
          x[i + h] = a - b;
        }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      x[i] = xlane_butterfly<16>(x[i], lane);
      x[i] = xlane_butterfly<32>(x[i], lane);
      x[i] *= 0.0625f;
    }
  }
  if constexpr (C == C_E2G16) divide_by_tensor_scale(x, v_scale);
  uint32_t cd[N];  // code of element k in the low BITS bits
  if constexpr (C == C_F16) {
#pragma unroll
    for (int k = 0; k < N; ++k) cd[k] = f16_bits(x[k]);
  } else if constexpr (C == C_E4TEN) {
    const float s = v_scale, r = __fdiv_rn(1.0f, s);
    const bool fast = s >= 0x1p-30f && s <= 0x1p30f;  // uniform
#pragma unroll
    for (int k = 0; k < N; ++k) cd[k] = token_code<C>(token_quot<C>(x[k], s, r, 0u, fast));
  } else {
    // a group is NTG whole n-tiles (a row: all of them): the lane's NTG
    // elements of it, then the 16 (row: 64) lanes that hold its columns
    constexpr int GS = codec_group(C) < 0 ? D : codec_group(C);
    constexpr int NTG = GS / 16 < N ? GS / 16 : N;  // a group's elements in one lane
    constexpr int GPL = N / NTG;                    // groups per lane
    constexpr int G = D / GS;
    uint32_t sb[GPL];
#pragma unroll
    for (int gl = 0; gl < GPL; ++gl) {
      float am = abs_max<NTG>(x + gl * NTG);
      am = GS == D ? max_over_lanes_wave<64>(am) : max_over_lanes_wave<16>(am);
      float s, r;
      group_scale<C>(am, s, r, sb[gl]);
      const bool zero = !mx_scaled(C) && !(s > 0.0f);
#pragma unroll
      for (int k = gl * NTG; k < gl * NTG + NTG; ++k)
        cd[k] = zero ? 0u : token_code<C>(token_quot<C>(x[k], s, r, sb[gl], true));
    }
    // lane n < GPL of each lane row stores the scale of its group n (a row
    // scale: lane 0)
    uint32_t mine = sb[0];
#pragma unroll
    for (int gl = 1; gl < GPL; ++gl) mine = n == gl ? sb[gl] : mine;
    if (n < GPL && (GS < D || Q == 0)) {
      const int grp = GS == D ? 0 : (N * Q) / NTG + n;
      if constexpr (BITS == 4) scales[gv * 4 * G + grp * 4 + te] = (uint8_t)mine;
      else if constexpr (scale_bytes(C) == 2) *reinterpret_cast<uint16_t*>(scales + (t * G + grp) * 2) = (uint16_t)mine;
      else scales[t * G + grp] = (uint8_t)mine;
    }
  }
  if constexpr (BITS == 4) {
    // the lane's nibbles of n-tiles 4 Q + k (k < 4) lie in one 8-byte word of
    // tile row gv * 16 + n, 16 bits apart
    static_assert(N == 4, "4-bit V planes are 256 wide");
    const int st = 8 * (te >> 1) + 4 * (te & 1);
    uint64_t v = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) v |= (uint64_t)cd[k] << (16 * k);
    const uint64_t mask = 0x000F000F000F000Full << st;
    unsigned long long* wp =
        reinterpret_cast<unsigned long long*>(codes + (Q >> 1) * 1024 + (gv * 16 + n) * 16 + (Q & 1) * 8);
    atomicAnd(wp, ~mask);
    atomicOr(wp, v << st);
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const int jt = N * Q + k;
      if constexpr (BITS == 8) codes[(jt >> 2) * 1024 + (gv * 16 + n) * 16 + (jt & 3) * 4 + te] = (uint8_t)cd[k];
      else *reinterpret_cast<uint16_t*>(codes + (jt >> 1) * 1024 + (gv * 16 + n) * 16 + (jt & 1) * 8 + 2 * te) =
               (uint16_t)cd[k];
    }
  }
}

}  // namespace enc
}  // namespace kvq
