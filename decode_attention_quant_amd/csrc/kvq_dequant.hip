// kvq_dequant.hip -- decode one physical page back to fp32.
//
// The stored value of an element is code x scale of its group, which is
// exact in fp32 for every format but FP8_TENSOR (one rounding of code x
// k_scale); no other rounding is added (the llama.cpp FP8-KV article names
// extra rounding when caches move as a quality risk).  Without
// KVQ_DEQUANT_STORED_DOMAIN, rotated planes are mapped back with H y / 16.
//
// One wave per (token, kv head, plane); lane l holds elements E*l .. E*l+E-1.
#include <hip/hip_runtime.h>

#include "kvq_device.hpp"
#include "kvq_internal.hpp"

namespace kvq {

template <int C, int PLANE, int D>
__device__ __forceinline__ float stored_value(const uint8_t* codes, const uint8_t* scales, int t, int d,
                                              float tensor_scale) {
  constexpr int BITS = codec_bits(C);
  uint32_t code;
  if constexpr (PLANE == 0) {
    const int byte = k_code_byte(BITS, t, d);
    if constexpr (BITS == 16) code = *reinterpret_cast<const uint16_t*>(codes + byte);
    else if constexpr (BITS == 8) code = codes[byte];
    else code = (codes[byte] >> (((d & 7) & 1) * 4)) & 0xFu;
  } else {
    const int g = t >> 2, e = t & 3, jt = d >> 4, n = d & 15;
    if constexpr (BITS == 16)
      code = *reinterpret_cast<const uint16_t*>(codes + (jt >> 1) * 1024 + (g * 16 + n) * 16 + (jt & 1) * 8 + 2 * e);
    else if constexpr (BITS == 8)
      code = codes[(jt >> 2) * 1024 + (g * 16 + n) * 16 + (jt & 3) * 4 + e];
    else
      code = (codes[(jt >> 3) * 1024 + (g * 16 + n) * 16 + (jt & 7) * 2 + (e >> 1)] >> ((e & 1) * 4)) & 0xFu;
  }
  if constexpr (C == C_BF16) return bf16_to_f32(code);
  if constexpr (C == C_F16) return f16_bits_to_f32(code);
  if constexpr (C == C_E4TEN) return e4m3_value(code) * tensor_scale;
  constexpr int G = n_groups(C, D);
  const int grp = codec_group(C) < 0 ? 0 : d / codec_group(C);
  if constexpr (C == C_I8G64 || C == C_E4ROW) {
    const float s = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(scales + (t * G + grp) * 2));
    const float c = C == C_I8G64 ? (float)(int8_t)(uint8_t)code : e4m3_value(code);
    return c * s;
  } else if constexpr (C == C_E2G16) {
    const int pos = PLANE == 1 ? ((t >> 2) * 4 * G + grp * 4 + (t & 3)) : (t * G + grp);
    const float s = e4m3_value(scales[pos]);
    const float mag[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
    const float c = (code & 8) ? -mag[code & 7] : mag[code & 7];
    return c * s * tensor_scale;  // exact: the two-level form's scale, 1 for single level
  } else if constexpr (C == C_E2MX) {
    const int pos = PLANE == 1 ? ((t >> 2) * 4 * G + grp * 4 + (t & 3)) : (t * G + grp);
    const float mag[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
    const float c = (code & 8) ? -mag[code & 7] : mag[code & 7];
    return ldexpf(c, (int)scales[pos] - 127);
  } else {  // C_E4MX
    return ldexpf(e4m3_value(code), (int)scales[t * G + grp] - 127);
  }
}

template <int FMT, int D>
__global__ __launch_bounds__(256) void dequant_page_kernel(Geometry geo, const uint8_t* __restrict__ pool,
                                                           int64_t page, int stored, float k_scale, float v_scale,
                                                           float* __restrict__ k_out, float* __restrict__ v_out) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // (head * P + slot) * 2 + plane
  if (row >= geo.H_kv * geo.P * 2) return;
  const int plane = row & 1;
  const int hs = row >> 1;
  const int head = hs / geo.P, slot = hs - head * geo.P;
  const int blk = slot >> 4, t = slot & 15;
  const uint8_t* hb = pool + page * geo.page_bytes + (int64_t)head * geo.head_bytes;
  float x[E];
  bool rot;
  if (plane == 0) {
    const uint8_t* c = hb + geo.off_kc + (int64_t)blk * geo.kcode_blk;
    const uint8_t* s = hb + geo.off_ks + (int64_t)blk * geo.kscale_blk;
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] = stored_value<k_codec(FMT), 0, D>(c, s, t, E * lane + i, k_scale);
    rot = k_rotated(FMT);
  } else {
    const uint8_t* c = hb + geo.off_vc + (int64_t)blk * geo.vcode_blk;
    const uint8_t* s = hb + geo.off_vs + (int64_t)blk * geo.vscale_blk;
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] = stored_value<v_codec(FMT), 1, D>(c, s, t, E * lane + i, v_scale);
    rot = v_rotated(FMT);
  }
  if (rot && !stored) {
    // H y / 16 over 64 lanes x E values (read path: any fp32 order)
#pragma unroll
    for (int hh = 1; hh < E; hh <<= 1)
#pragma unroll
      for (int i = 0; i < E; ++i)
        if ((i & hh) == 0) {
          const float a = x[i], b = x[i + hh];
          x[i] = a + b;
          x[i + hh] = a - b;
        }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const bool upper = (lane & m) != 0;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const float p = __shfl_xor(x[i], m);
        x[i] = upper ? (p - x[i]) : (x[i] + p);
      }
    }
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] *= 0.0625f;
  }
  float* dst = (plane == 0 ? k_out : v_out) + ((int64_t)head * geo.P + slot) * D + E * lane;
#pragma unroll
  for (int i = 0; i < E; ++i) dst[i] = x[i];
}

template <int FMT, int D>
static hipError_t launch_dq_t(const Geometry& geo, const uint8_t* pool, int64_t page, bool stored, float ks,
                              float vs, float* ko, float* vo, hipStream_t stream) {
  const int rows = geo.H_kv * geo.P * 2;
  hipLaunchKernelGGL((dequant_page_kernel<FMT, D>), dim3((rows + 3) / 4), dim3(256), 0, stream, geo, pool, page,
                     stored ? 1 : 0, ks, vs, ko, vo);
  return hipGetLastError();
}

hipError_t launch_dequant_page(const Geometry& geo, const uint8_t* pool, int64_t page, bool stored, float ks,
                               float vs, float* ko, float* vo, hipStream_t stream) {
#define KVQ_DQ_CASE(F, DD) \
  if (geo.fmt == F && geo.D == DD) return launch_dq_t<F, DD>(geo, pool, page, stored, ks, vs, ko, vo, stream);
  KVQ_DQ_CASE(F_BF16, 128) KVQ_DQ_CASE(F_BF16, 256)
  KVQ_DQ_CASE(F_FP8_ROW, 128) KVQ_DQ_CASE(F_FP8_ROW, 256)
  KVQ_DQ_CASE(F_FP8_TENSOR, 128) KVQ_DQ_CASE(F_FP8_TENSOR, 256)
  KVQ_DQ_CASE(F_MXFP8, 128) KVQ_DQ_CASE(F_MXFP8, 256)
  KVQ_DQ_CASE(F_INT8_G64, 256) KVQ_DQ_CASE(F_NVFP4_G16, 256) KVQ_DQ_CASE(F_K8V4, 256)
  KVQ_DQ_CASE(F_MXFP4, 256)
#undef KVQ_DQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
