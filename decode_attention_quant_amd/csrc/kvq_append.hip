// kvq_append.hip -- quantize-append: encode bf16 K/V rows and store them in
// the paged pool (the write path of every format of the NInfer KV-cache
// quantization guide, section on the five formats; TokenSpeed mxfp8 and
// fp8_e4m3; Qwen FP8-KV article's per-tensor symmetric FP8).
//
// Work split: 16 lanes encode one row (one token, one kv head, one plane);
// a wave encodes 4 rows of the same plane, so every lane of a wave runs the
// same codec.  Lane j of a row holds elements [j*D/16, (j+1)*D/16).
#include <hip/hip_runtime.h>

#include "kvq_device.hpp"
#include "kvq_internal.hpp"

namespace kvq {

// Encode EPL consecutive values of one row (this lane's share) with codec C,
// group maxima reduced over the lanes that share a group, then store codes
// and scales at their tiled positions.
template <int C, int D, bool ROT, int PLANE>
__device__ __forceinline__ void encode_store(float (&x)[D / 16], int lane16, uint8_t* codes, uint8_t* scales,
                                             int t, float tensor_scale) {
  constexpr int EPL = D / 16;
  constexpr int BITS = codec_bits(C);
  if constexpr (ROT) {
    static_assert(D == 256, "the rotation is 256-point");
    fwht256_rows16(x, lane16);
  }

  uint32_t code[EPL];
  // ---------------------------------------------------------------- codes
  if constexpr (C == C_F16) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) code[i] = f16_bits(x[i]);
  } else if constexpr (C == C_E4TEN) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) code[i] = e4m3_code(__fdiv_rn(x[i], tensor_scale));
  } else {
    constexpr int GS = codec_group(C) < 0 ? D : codec_group(C);
    constexpr int LANES_PER_GROUP = GS / EPL > 0 ? GS / EPL : 1;  // lanes sharing one group
    constexpr int GROUPS_PER_LANE = EPL / GS > 0 ? EPL / GS : 1;
    constexpr int G = D / GS;
    float amax[GROUPS_PER_LANE];
#pragma unroll
    for (int gl = 0; gl < GROUPS_PER_LANE; ++gl) {
      float a = 0.0f;
      constexpr int PER = EPL / GROUPS_PER_LANE;
#pragma unroll
      for (int i = 0; i < PER; ++i) a = fmaxf(a, fabsf(x[gl * PER + i]));
#pragma unroll
      for (int m = 1; m < LANES_PER_GROUP; m <<= 1) a = fmaxf(a, shfl_xor16(a, m));
      amax[gl] = a;
    }
#pragma unroll
    for (int gl = 0; gl < GROUPS_PER_LANE; ++gl) {
      constexpr int PER = EPL / GROUPS_PER_LANE;
      const int grp = (lane16 * EPL) / GS + gl;  // group index of this run
      const bool first = ((lane16 * EPL) % GS) == 0;
      uint32_t sbits;
      float s;
      if constexpr (C == C_I8G64 || C == C_E4ROW) {
        sbits = f16_scale_bits(__fdiv_rn(amax[gl], C == C_I8G64 ? 127.0f : 448.0f));
        s = f16_bits_to_f32(sbits);
      } else if constexpr (C == C_E2G16) {
        sbits = e4m3_code(__fdiv_rn(amax[gl], 6.0f));  // amax >= 0: sign bit stays 0
        s = e4m3_value(sbits);
      } else {  // C_E4MX: OCP MX shared exponent floor(log2 amax) - 8, biased by 127
        const int e = __builtin_amdgcn_frexp_expf(amax[gl]) - 1;
        int b = e - 8 + 127;
        b = b < 0 ? 0 : (b > 254 ? 254 : b);
        sbits = amax[gl] > 0.0f ? (uint32_t)b : 0u;
        s = ldexpf(1.0f, (int)sbits - 127);  // exact power of two (2^-127 is subnormal)
      }
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const float v = x[gl * PER + i];
        uint32_t c;
        if constexpr (C == C_I8G64) {
          const float q = rintf(__fdiv_rn(v, s));
          const int iq = (int)fmaxf(fminf(q, 127.0f), -127.0f);
          c = (s == 0.0f) ? 0u : ((uint32_t)iq & 0xFFu);
        } else if constexpr (C == C_E4ROW) {
          c = (s == 0.0f) ? 0u : e4m3_code(__fdiv_rn(v, s));
        } else if constexpr (C == C_E2G16) {
          c = (s == 0.0f) ? 0u : e2m1_code(__fdiv_rn(v, s));
        } else {
          c = e4m3_code(__fdiv_rn(v, s));
        }
        code[gl * PER + i] = c;
      }
      if (first) {
        if constexpr (scale_bytes(C) == 2) {
          uint8_t* sp = scales + (t * G + grp) * 2;
          *reinterpret_cast<uint16_t*>(sp) = (uint16_t)sbits;
        } else {
          int pos = (PLANE == 1 && C == C_E2G16) ? ((t >> 2) * 4 * G + grp * 4 + (t & 3)) : (t * G + grp);
          scales[pos] = (uint8_t)sbits;
        }
      }
    }
  }

  // ---------------------------------------------------------------- store codes
  const int d0 = lane16 * EPL;
  if constexpr (PLANE == 0) {
    // K: runs of 8 consecutive d share one contiguous span of the tile
#pragma unroll
    for (int r = 0; r < EPL / 8; ++r) {
      const int d = d0 + 8 * r;
      uint8_t* p = codes + k_code_byte(BITS, t, d);
      if constexpr (BITS == 16) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = code[8 * r + 2 * i] | (code[8 * r + 2 * i + 1] << 16);
        *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
      } else if constexpr (BITS == 8) {
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w0 |= code[8 * r + i] << (8 * i);
          w1 |= code[8 * r + 4 + i] << (8 * i);
        }
        *reinterpret_cast<uint2*>(p) = make_uint2(w0, w1);
      } else {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) w |= code[8 * r + i] << (4 * i);
        *reinterpret_cast<uint32_t*>(p) = w;
      }
    }
  } else {
    // V: token t = 4g + e; element (t, d = 16*jt + n)
    const int g = t >> 2, e = t & 3;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int d = d0 + i;
      const int jt = d >> 4, n = d & 15;
      if constexpr (BITS == 8) {
        codes[(jt >> 2) * 1024 + (g * 16 + n) * 16 + (jt & 3) * 4 + e] = (uint8_t)code[i];
      } else if constexpr (BITS == 16) {
        *reinterpret_cast<uint16_t*>(codes + (jt >> 1) * 1024 + (g * 16 + n) * 16 + (jt & 1) * 8 + 2 * e) =
            (uint16_t)code[i];
      } else {
        // this lane holds all 16 n of its n-tile: pair n with n + 8 into one byte
        if (n < 8)
          codes[(jt >> 2) * 512 + (g * 8 + n) * 16 + (jt & 3) * 4 + e] = (uint8_t)(code[i] | (code[i + 8] << 4));
      }
    }
  }
}

template <int FMT, int D>
__global__ __launch_bounds__(256) void append_kernel(uint8_t* __restrict__ pool, const uint16_t* __restrict__ k,
                                                     const uint16_t* __restrict__ v, int64_t num_rows,
                                                     const int32_t* __restrict__ slots, Geometry geo,
                                                     float k_scale, float v_scale) {
  constexpr int EPL = D / 16;
  const int wave = threadIdx.x >> 6;
  const int lane16 = threadIdx.x & 15;
  const int64_t gw = (int64_t)blockIdx.x * 4 + wave;  // global wave
  const int plane = (int)(gw & 1);
  const int64_t row = (gw >> 1) * 4 + ((threadIdx.x & 63) >> 4);  // token * H_kv + head
  if (row >= num_rows) return;
  const int64_t token = row / geo.H_kv;
  const int head = (int)(row - token * geo.H_kv);
  const int slot = slots[token];
  if (slot < 0) return;
  const int64_t page = slot / geo.P;
  const int off = slot - (int)(page * geo.P);
  const int blk = off >> 4, t = off & 15;
  uint8_t* head_base = pool + page * geo.page_bytes + (int64_t)head * geo.head_bytes;

  const uint16_t* src = (plane ? v : k) + row * D + lane16 * EPL;
  uint32_t raw[EPL / 2];
#pragma unroll
  for (int i = 0; i < EPL / 8; ++i) {
    const uint4 w = *reinterpret_cast<const uint4*>(src + 8 * i);
    raw[4 * i] = w.x; raw[4 * i + 1] = w.y; raw[4 * i + 2] = w.z; raw[4 * i + 3] = w.w;
  }

  constexpr int KC = k_codec(FMT), VC = v_codec(FMT);
  if (plane == 0) {
    uint8_t* codes = head_base + geo.off_kc + (int64_t)blk * geo.kcode_blk;
    uint8_t* scales = head_base + geo.off_ks + (int64_t)blk * geo.kscale_blk;
    if constexpr (KC == C_BF16) {
      // K of BF16 is stored bit for bit
#pragma unroll
      for (int r = 0; r < EPL / 8; ++r) {
        uint8_t* p = codes + k_code_byte(16, t, lane16 * EPL + 8 * r);
        *reinterpret_cast<uint4*>(p) = make_uint4(raw[4 * r], raw[4 * r + 1], raw[4 * r + 2], raw[4 * r + 3]);
      }
    } else {
      float x[EPL];
#pragma unroll
      for (int i = 0; i < EPL / 2; ++i) {
        x[2 * i] = bf16_to_f32(raw[i] & 0xFFFFu);
        x[2 * i + 1] = bf16_to_f32(raw[i] >> 16);
      }
      encode_store<KC, D, k_rotated(FMT), 0>(x, lane16, codes, scales, t, k_scale);
    }
  } else {
    uint8_t* codes = head_base + geo.off_vc + (int64_t)blk * geo.vcode_blk;
    uint8_t* scales = head_base + geo.off_vs + (int64_t)blk * geo.vscale_blk;
    float x[EPL];
#pragma unroll
    for (int i = 0; i < EPL / 2; ++i) {
      x[2 * i] = bf16_to_f32(raw[i] & 0xFFFFu);
      x[2 * i + 1] = bf16_to_f32(raw[i] >> 16);
    }
    encode_store<VC, D, v_rotated(FMT), 1>(x, lane16, codes, scales, t, v_scale);
  }
}

template <int FMT, int D>
static hipError_t launch_append_t(uint8_t* pool, const uint16_t* k, const uint16_t* v, int64_t T,
                                  const int32_t* slots, const Geometry& geo, float ks, float vs,
                                  hipStream_t stream) {
  const int64_t rows = T * geo.H_kv;
  const int64_t waves = 2 * ((rows + 3) / 4);
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((append_kernel<FMT, D>), dim3((unsigned)blocks), dim3(256), 0, stream, pool, k, v, rows,
                     slots, geo, ks, vs);
  return hipGetLastError();
}

hipError_t launch_append(uint8_t* pool, const uint16_t* k, const uint16_t* v, int64_t T, const int32_t* slots,
                         const Geometry& geo, float ks, float vs, hipStream_t stream) {
#define KVQ_APPEND_CASE(F, DD) \
  if (geo.fmt == F && geo.D == DD) return launch_append_t<F, DD>(pool, k, v, T, slots, geo, ks, vs, stream);
  KVQ_APPEND_CASE(F_BF16, 128) KVQ_APPEND_CASE(F_BF16, 256)
  KVQ_APPEND_CASE(F_FP8_ROW, 128) KVQ_APPEND_CASE(F_FP8_ROW, 256)
  KVQ_APPEND_CASE(F_FP8_TENSOR, 128) KVQ_APPEND_CASE(F_FP8_TENSOR, 256)
  KVQ_APPEND_CASE(F_MXFP8, 128) KVQ_APPEND_CASE(F_MXFP8, 256)
  KVQ_APPEND_CASE(F_INT8_G64, 256) KVQ_APPEND_CASE(F_NVFP4_G16, 256) KVQ_APPEND_CASE(F_K8V4, 256)
#undef KVQ_APPEND_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
