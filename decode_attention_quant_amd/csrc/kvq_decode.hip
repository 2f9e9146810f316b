// kvq_decode.hip -- split-K decode attention over the compressed paged cache.
//
// Every decode step reads all cached K/V of each sequence, so the bytes
// stored per token set the speed (NInfer KV-cache guide, section on why the
// cache is quantized; Qwen FP8-KV article, bandwidth section).  This kernel
// therefore streams each page plane exactly once with 16-byte loads and does
// the rest in registers:
//
//  grid (split s + nsplit * unit u, row tile), u = b * H_kv + h: one workgroup of 4 waves
//  walks pages [s*pps, (s+1)*pps) of sequence b, kv head h.  The rows of the
//  workgroup are the R = G * n_q query rows sharing that kv head (GQA group
//  times MTP tokens, up to 16 per tile).  Wave w takes token blocks
//  w, w+4, ... (16 tokens each) and keeps its own online-softmax state.
//
//  per token block (one wave):
//    S (16 tokens x 16 rows) = K_blk . Q^T with v_mfma_f32_16x16x32_{bf16,f16}:
//      K codes are expanded to bf16 / f16 exactly (E4M3, int8 and
//      E2M1 x UE4M3 values are exact there); row / group scales multiply
//      the fp32 partial sums; rotated formats use Q' = H q / 16 split into
//      f16 hi + lo parts (two MFMAs) so q keeps ~22 bits.
//    online softmax in base 2 (exp2), masking t >= L and the MTP causal rule.
//    O (16 rows x D) += P . V_blk with v_mfma_f32_16x16x16_f16; V codes are
//      expanded to f16 with their scale folded in (one rounding).
//  The 4 waves merge through LDS; the workgroup writes either partial
//  (m, l, o) for the combine kernel, or, with one split per sequence, the
//  normalized output directly (un-rotating V for NVFP4 / K8V4).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kvq_device.hpp"
#include "kvq_internal.hpp"

namespace kvq {

template <int FMT, int D>
struct DT {
  static constexpr int KC = k_codec(FMT), VC = v_codec(FMT);
  static constexpr int KBITS = codec_bits(KC), VBITS = codec_bits(VC);
  static constexpr bool QF16 = k_rotated(FMT);  // rotated q -> f16 hi/lo
  static constexpr bool VROT = v_rotated(FMT);
  static constexpr int KSTEPS = D / 32;
  static constexpr int NT = D / 16;
  static constexpr int KCH = D * KBITS / 512;                       // 16-B K chunks per lane per block
  static constexpr int VCH = (VBITS == 16 ? 2 : 1) * NT * 4 / 16;   // 16-B V chunks per lane per block
  static constexpr int KSW = KC == C_E4ROW ? 2 : KC == C_I8G64 ? 8 : KC == C_E4MX ? D / 32 : KC == C_E2G16 ? 4 : 0;
  static constexpr int VSW = VC == C_E4ROW ? 2 : VC == C_I8G64 ? 8 : VC == C_E4MX ? D / 32 : VC == C_E2G16 ? 16 : 0;
  static constexpr int G = n_groups(KC, D) > 0 ? n_groups(KC, D) : 1;
};

template <int FMT, int D>
struct Buf {
  uint4 k[DT<FMT, D>::KCH];
  uint4 v[DT<FMT, D>::VCH];
  uint32_t ks[DT<FMT, D>::KSW > 0 ? DT<FMT, D>::KSW : 1];
  uint32_t vs[DT<FMT, D>::VSW > 0 ? DT<FMT, D>::VSW : 1];
};

template <int N>
__device__ __forceinline__ void load_words(uint32_t (&w)[N], const uint8_t* p) {
  if constexpr (N == 2) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    w[0] = x.x; w[1] = x.y;
  } else {
    static_assert(N % 4 == 0, "");
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint4 x = *reinterpret_cast<const uint4*>(p + 16 * i);
      w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
    }
  }
}

// Load token block j of this split into registers.
template <int FMT, int D>
__device__ __forceinline__ void load_block(Buf<FMT, D>& buf, const uint8_t* head0, const Geometry& geo,
                                           const int32_t* bt_row, int page0, int j, int lane) {
  using T = DT<FMT, D>;
  const int bpp = geo.P >> 4;
  const int page = page0 + j / bpp;
  const int bip = j - (j / bpp) * bpp;
  const int64_t phys = bt_row[page];
  const uint8_t* hb = head0 + phys * geo.page_bytes;
  const int g = lane >> 4, c16 = lane & 15;
  const uint8_t* kc = hb + geo.off_kc + (int64_t)bip * geo.kcode_blk;
  const uint8_t* vc = hb + geo.off_vc + (int64_t)bip * geo.vcode_blk;
#pragma unroll
  for (int i = 0; i < T::KCH; ++i) buf.k[i] = *reinterpret_cast<const uint4*>(kc + i * 1024 + lane * 16);
#pragma unroll
  for (int q = 0; q < T::VCH; ++q) {
    if constexpr (T::VBITS == 4)
      buf.v[q] = *reinterpret_cast<const uint4*>(vc + q * 512 + (g * 8 + (c16 & 7)) * 16);
    else
      buf.v[q] = *reinterpret_cast<const uint4*>(vc + q * 1024 + lane * 16);
  }
  if constexpr (T::KSW > 0) {
    const uint8_t* ks = hb + geo.off_ks + (int64_t)bip * geo.kscale_blk;
    const int off = T::KC == C_E2G16 ? c16 * 16 : g * (4 * T::KSW);
    load_words(buf.ks, ks + off);
  }
  if constexpr (T::VSW > 0) {
    const uint8_t* vs = hb + geo.off_vs + (int64_t)bip * geo.vscale_blk;
    load_words(buf.vs, vs + g * (4 * T::VSW));
  }
}

// ----------------------------------------------------------- operand expanders

// 8 E4M3 codes (two dwords) -> bf16x8, exact
__device__ __forceinline__ bf16x8 e4m3x8_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 4 signed int8 codes -> 2 x f16x2, exact: the byte with its sign bit
// flipped (c + 128) becomes the low mantissa of 1024, then 1152 is removed.
__device__ __forceinline__ void i8x4_f16(uint32_t w, f16x2& lo, f16x2& hi) {
  const uint32_t u = w ^ 0x80808080u;
  const f16x2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  lo = bitcast<f16x2>(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) + bias;
  hi = bitcast<f16x2>(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) + bias;
}

__device__ __forceinline__ f16x8 i8x8_f16(uint32_t w0, uint32_t w1) {
  f16x2 a, b, c, d;
  i8x4_f16(w0, a, b);
  i8x4_f16(w1, c, d);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 8 E2M1 codes (one dword, element e in nibble e) -> f16x8, exact
__device__ __forceinline__ f16x8 e2m1x8_f16(uint32_t w) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ uint32_t word(const uint4& q, int i) {
  return i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w;
}

// ----------------------------------------------------------- Q operands

template <int FMT, int D>
struct QOps {
  // B operands of S = K . Q^T per k-step: bf16 (plain q) or f16 hi/lo (rotated q)
  typename std::conditional<DT<FMT, D>::QF16, f16x8, bf16x8>::type hi[DT<FMT, D>::KSTEPS];
  f16x8 lo[DT<FMT, D>::QF16 ? DT<FMT, D>::KSTEPS : 1];
};

// ----------------------------------------------------------- S = K . Q^T

template <int FMT, int D>
__device__ __forceinline__ f32x4 qk_block(const Buf<FMT, D>& buf, const QOps<FMT, D>& qo, int lane) {
  using T = DT<FMT, D>;
  f32x4 S = {0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  if constexpr (T::KC == C_BF16) {
#pragma unroll
    for (int kk = 0; kk < T::KSTEPS; ++kk)
      S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(buf.k[kk]), qo.hi[kk], S, 0, 0, 0);
  } else if constexpr (T::KC == C_E4ROW || T::KC == C_E4TEN) {
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) {
      S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_bf16(buf.k[i].x, buf.k[i].y), qo.hi[2 * i], S, 0, 0, 0);
      S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_bf16(buf.k[i].z, buf.k[i].w), qo.hi[2 * i + 1], S, 0, 0, 0);
    }
    if constexpr (T::KC == C_E4ROW) {
      // one fp16 scale per token: tokens 4g..4g+3 in ks[0] (lo, hi), ks[1]
      S[0] *= f16_bits_to_f32(buf.ks[0] & 0xFFFFu);
      S[1] *= f16_bits_to_f32(buf.ks[0] >> 16);
      S[2] *= f16_bits_to_f32(buf.ks[1] & 0xFFFFu);
      S[3] *= f16_bits_to_f32(buf.ks[1] >> 16);
    }
  } else if constexpr (T::KC == C_E4MX) {
    // one UE8M0 per 32 values = per k-step: scale each k-step's partial sum
    constexpr int G = D / 32;
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int kk = 2 * i + hh;
        const f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            e4m3x8_bf16(hh ? buf.k[i].z : buf.k[i].x, hh ? buf.k[i].w : buf.k[i].y), qo.hi[kk], zero, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int bi = e * G + kk;  // token 4g+e, group kk
          const int ex = (int)((buf.ks[bi >> 2] >> (8 * (bi & 3))) & 0xFFu) - 127;
          S[e] += ldexpf(acc[e], ex);
        }
      }
    }
  } else if constexpr (T::KC == C_I8G64) {
    // one fp16 scale per 64 values = two k-steps = one chunk
#pragma unroll
    for (int grp = 0; grp < T::KCH; ++grp) {
      const f16x8 a0 = i8x8_f16(buf.k[grp].x, buf.k[grp].y);
      const f16x8 a1 = i8x8_f16(buf.k[grp].z, buf.k[grp].w);
      f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qo.hi[2 * grp], zero, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qo.lo[2 * grp], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qo.hi[2 * grp + 1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qo.lo[2 * grp + 1], acc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int hw = e * 4 + grp;  // halfword of token 4g+e, group grp
        S[e] += acc[e] * f16_bits_to_f32((buf.ks[hw >> 1] >> (16 * (hw & 1))) & 0xFFFFu);
      }
    }
  } else if constexpr (T::KC == C_E2G16) {
    // E2M1 x UE4M3 is exact in f16: fold the group scale into the operand.
    // lane (g, t): k-step kk covers d in [32kk + 8g, +8) -> group 2kk + g/2
    const int gb = (lane >> 5) & 1;
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) {
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        const int kk = 4 * i + hh;
        const uint32_t sw = buf.ks[kk >> 1];
        const uint32_t sb = (sw >> (8 * (2 * (kk & 1) + gb))) & 0xFFu;
        const _Float16 s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)sb, 1.0f, false)[0];
        f16x8 a = e2m1x8_f16(word(buf.k[i], hh));
        a *= s;
        S = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qo.hi[kk], S, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qo.lo[kk], S, 0, 0, 0);
      }
    }
  }
  return S;
}

// ----------------------------------------------------------- V operands

// B operand of O += P . V for n-tile nt: tokens 4g..4g+3 of column 16*nt + n.
template <int FMT, int D>
__device__ __forceinline__ f16x4 v_operand(const Buf<FMT, D>& buf, int nt, int lane) {
  using T = DT<FMT, D>;
  if constexpr (T::VC == C_F16) {
    const uint4& q = buf.v[nt >> 1];
    const uint32_t a = (nt & 1) ? q.z : q.x, b = (nt & 1) ? q.w : q.y;
    return bitcast<f16x4>(make_uint2(a, b));
  } else if constexpr (T::VC == C_E4ROW || T::VC == C_E4TEN || T::VC == C_E4MX) {
    const uint32_t w = word(buf.v[nt >> 2], nt & 3);
    if constexpr (T::VC == C_E4MX) {
      // UE8M0 per (token, 32 values): code * 2^e in fp32, one RNE to f16
      constexpr int G = D / 32;
      const int grp = nt >> 1;
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
      float x[4] = {lo[0], lo[1], hi[0], hi[1]};
      f16x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int bi = e * G + grp;
        const int ex = (int)((buf.vs[bi >> 2] >> (8 * (bi & 3))) & 0xFFu) - 127;
        r[e] = (_Float16)ldexpf(x[e], ex);
      }
      return r;
    } else {
      f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, false);
      f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, true);
      if constexpr (T::VC == C_E4ROW) {
        a *= bitcast<f16x2>(buf.vs[0]);
        b *= bitcast<f16x2>(buf.vs[1]);
      }
      return f16x4{a[0], a[1], b[0], b[1]};
    }
  } else if constexpr (T::VC == C_I8G64) {
    const uint32_t w = word(buf.v[nt >> 2], nt & 3);
    f16x2 a, b;
    i8x4_f16(w, a, b);
    // scales: halfword (e*4 + grp) of vs; pair tokens (0,1) and (2,3)
    const int grp = nt >> 2;
    const uint32_t sel = (grp & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t s01 = __builtin_amdgcn_perm(buf.vs[2 + (grp >> 1)], buf.vs[grp >> 1], sel);
    const uint32_t s23 = __builtin_amdgcn_perm(buf.vs[6 + (grp >> 1)], buf.vs[4 + (grp >> 1)], sel);
    a *= bitcast<f16x2>(s01);
    b *= bitcast<f16x2>(s23);
    return f16x4{a[0], a[1], b[0], b[1]};
  } else {  // C_E2G16: byte e holds (token 4g+e, n) low and (token 4g+e, n+8) high
    const uint32_t w = word(buf.v[nt >> 2], nt & 3);
    const uint32_t x = (w >> (((lane & 15) >= 8) ? 4 : 0)) & 0x0F0F0F0Fu;
    const uint32_t y = x | (x >> 4);  // byte 0: t0 | t1 << 4, byte 2: t2 | t3 << 4
    f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y, 1.0f, 0);
    f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y, 1.0f, 2);
    const uint32_t sw = buf.vs[nt];  // UE4M3 of tokens 4g..4g+3, group nt
    a *= __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)sw, 1.0f, false);
    b *= __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)sw, 1.0f, true);
    return f16x4{a[0], a[1], b[0], b[1]};
  }
}

// ----------------------------------------------------------- 64-lane FWHT
// Unnormalized-order-free Hadamard (any fp32 order is fine on the read
// path): lane l holds elements E*l .. E*l+E-1 of a 64*E vector.
template <int E>
__device__ __forceinline__ void fwht_wave(float (&x)[E], int lane) {
#pragma unroll
  for (int h = 1; h < E; h <<= 1)
#pragma unroll
    for (int i = 0; i < E; ++i)
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
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
}

// ----------------------------------------------------------- the kernel

template <int FMT, int D>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(Geometry geo, DecodeArgs a) {
  using T = DT<FMT, D>;
  constexpr float NEG_INF = -__builtin_inff();
  __shared__ float lds[4 * 16 * D + 2 * 64 + 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int s = (int)(blockIdx.x % (unsigned)a.nsplit), u = (int)(blockIdx.x / (unsigned)a.nsplit);
  const int rt = blockIdx.y;
  const int b = u / geo.H_kv, h = u - b * geo.H_kv;
  const int L = a.seq_lens[b];
  const int npages = (L + geo.P - 1) / geo.P;
  const int page0 = s * a.pps;
  if (page0 >= npages && !a.direct) return;
  const int tok0 = page0 * geo.P;
  const int tok1 = min(L, (page0 + a.pps) * geo.P);
  const int nblk = tok1 > tok0 ? (tok1 - tok0 + 15) >> 4 : 0;
  const int Rt = min(16, a.R - 16 * rt);

  // ---- query rows of this tile: row r (= c16 in S layout) -> (i, head)
  const int r = c16;
  const int rr = 16 * rt + r;
  const bool row_ok = r < Rt;
  const int qi = rr / a.G, qh = h * a.G + (rr - qi * a.G);
  const int limit = L - a.n_q + qi;  // last visible position of this row
  float crow = a.qk_scale;

  QOps<FMT, D> qo;
  if constexpr (!T::QF16) {
    const uint16_t* qp = a.q + (((int64_t)b * a.n_q + qi) * a.H_q + qh) * D;
#pragma unroll
    for (int kk = 0; kk < T::KSTEPS; ++kk) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (row_ok) w = *reinterpret_cast<const uint4*>(qp + 32 * kk + 8 * g);
      qo.hi[kk] = bitcast<bf16x8>(w);
    }
  } else {
    // q' = H q / 16 in fp32, scaled by 2^(8 - e) so that max|q'| lies in
    // [128, 256), then split into f16 hi + lo (about 22 significant bits).
    float* qrot = lds;              // [16][D]
    float* qexp = lds + 16 * D;     // [16]
    constexpr int E = D / 64;
    for (int row = wave; row < Rt; row += 4) {
      const int rr2 = 16 * rt + row;
      const int i2 = rr2 / a.G, h2 = h * a.G + (rr2 - i2 * a.G);
      const uint16_t* qp = a.q + (((int64_t)b * a.n_q + i2) * a.H_q + h2) * D + E * lane;
      float x[E];
      const uint2 w = *reinterpret_cast<const uint2*>(qp);
      x[0] = bf16_to_f32(w.x & 0xFFFFu); x[1] = bf16_to_f32(w.x >> 16);
      x[2] = bf16_to_f32(w.y & 0xFFFFu); x[3] = bf16_to_f32(w.y >> 16);
      fwht_wave<E>(x, lane);
      float am = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) { x[i] *= 0.0625f; am = fmaxf(am, fabsf(x[i])); }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) am = fmaxf(am, __shfl_xor(am, m));
      const int ex = am > 0.f ? __builtin_amdgcn_frexp_expf(am) : 0;
#pragma unroll
      for (int i = 0; i < E; ++i) qrot[row * D + E * lane + i] = ldexpf(x[i], 8 - ex);
      if (lane == 0) qexp[row] = (float)ex;
    }
    __syncthreads();
    if (row_ok) crow = a.qk_scale * ldexpf(1.0f, (int)qexp[r] - 8);
#pragma unroll
    for (int kk = 0; kk < T::KSTEPS; ++kk) {
      f16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = row_ok ? qrot[r * D + 32 * kk + 8 * g + e] : 0.f;
        hi[e] = (_Float16)v;
        lo[e] = (_Float16)(v - (float)hi[e]);
      }
      qo.hi[kk] = hi;
      qo.lo[kk] = lo;
    }
    __syncthreads();
  }

  // ---- stream this wave's token blocks
  const uint8_t* head0 = a.pool + (int64_t)h * geo.head_bytes;
  const int32_t* bt_row = a.block_table + (int64_t)b * a.max_pages;
  float m_run = NEG_INF, l_run = 0.f;
  f32x4 O[T::NT];
#pragma unroll
  for (int nt = 0; nt < T::NT; ++nt) O[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const Buf<FMT, D>& buf, int j) {
    const int t0 = tok0 + 16 * j;
    const f32x4 S = qk_block<FMT, D>(buf, qo, lane);
    float sc[4];
    float bm = NEG_INF;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = t0 + 4 * g + e;
      sc[e] = (row_ok && t <= limit) ? S[e] * crow : NEG_INF;
      bm = fmaxf(bm, sc[e]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float m_new = fmaxf(m_run, bm);
    if (__any(m_new > m_run)) {
      const float corr = (m_new > m_run) ? exp2f(m_run - m_new) : 1.0f;
      l_run *= corr;
      float ce[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ce[e] = __shfl(corr, 4 * g + e);
#pragma unroll
      for (int nt = 0; nt < T::NT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) O[nt][e] *= ce[e];
      m_run = m_new;
    }
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = (sc[e] == NEG_INF) ? 0.f : exp2f(sc[e] - m_run);
      l_run += p[e];
    }
    const f16x4 P = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
    const bool tail = t0 + 16 > L;  // slots past the end may hold anything: zero their V
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) {
      f16x4 vb = v_operand<FMT, D>(buf, nt, lane);
      if (tail) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (t0 + 4 * g + e >= L) vb[e] = (_Float16)0.0f;
      }
      O[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(P, vb, O[nt], 0, 0, 0);
    }
  };

  {
    Buf<FMT, D> A, Bb;
    int j = wave;
    if (j < nblk) load_block<FMT, D>(A, head0, geo, bt_row, page0, j, lane);
    while (j < nblk) {
      if (j + 4 < nblk) load_block<FMT, D>(Bb, head0, geo, bt_row, page0, j + 4, lane);
      process(A, j);
      j += 4;
      if (j >= nblk) break;
      if (j + 4 < nblk) load_block<FMT, D>(A, head0, geo, bt_row, page0, j + 4, lane);
      process(Bb, j);
      j += 4;
    }
  }

  // ---- merge the 4 waves
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  float* sm_o = lds;                    // [4][16][D]
  float* sm_m = lds + 4 * 16 * D;       // [4][16]
  float* sm_l = sm_m + 64;              // [4][16]
  if (lane < 16) {
    sm_m[wave * 16 + lane] = m_run;
    sm_l[wave * 16 + lane] = l_run;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * g + e;
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w * 16 + row]);
    const float mw = sm_m[wave * 16 + row];
    const float f = (mw == NEG_INF) ? 0.f : exp2f(mw - M);
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) sm_o[(wave * 16 + row) * D + 16 * nt + c16] = O[nt][e] * f;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < Rt * D; idx += 256) {
    const int row = idx / D, d = idx - row * D;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) o += sm_o[(w * 16 + row) * D + d];
    sm_o[row * D + d] = o;  // wave-0 slot of this row; read by this thread only
  }
  __syncthreads();

  // ---- write: one wave per row
  constexpr int E = D / 64;
  for (int row = wave; row < Rt; row += 4) {
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w * 16 + row]);
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sm_m[w * 16 + row];
      l += (mw == NEG_INF) ? 0.f : exp2f(mw - M) * sm_l[w * 16 + row];
    }
    const int rr2 = 16 * rt + row;
    float x[E];
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] = sm_o[row * D + E * lane + i];
    if (!a.direct) {
      const int64_t prow = ((int64_t)u * a.nsplit + s) * a.R + rr2;
      float* op = a.ws_o + prow * D + E * lane;
#pragma unroll
      for (int i = 0; i < E; ++i) op[i] = x[i];
      if (lane == 0) {
        a.ws_ml[prow * 2] = M;
        a.ws_ml[prow * 2 + 1] = l;
      }
    } else {
      const float inv = l > 0.f ? a.v_out_scale / l : 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) x[i] *= inv;
      if constexpr (T::VROT) {
        fwht_wave<E>(x, lane);
#pragma unroll
        for (int i = 0; i < E; ++i) x[i] *= 0.0625f;
      }
      const int i2 = rr2 / a.G, h2 = h * a.G + (rr2 - i2 * a.G);
      const int64_t orow = ((int64_t)b * a.n_q + i2) * a.H_q + h2;
      float* op = a.out + orow * D + E * lane;
#pragma unroll
      for (int i = 0; i < E; ++i) op[i] = x[i];
      if (a.lse != nullptr && lane == 0)
        a.lse[orow] = l > 0.f ? (M + __log2f(l)) * 0.69314718055994531f : NEG_INF;
    }
  }
}

// ----------------------------------------------------------- combine

template <int D, bool VROT>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a, int P, int H_kv) {
  constexpr float NEG_INF = -__builtin_inff();
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t rowid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nrows = (int64_t)a.B * H_kv * a.R;
  if (rowid >= nrows) return;
  const int u = (int)(rowid / a.R), rr = (int)(rowid - (int64_t)u * a.R);
  const int b = u / H_kv, h = u - b * H_kv;
  const int L = a.seq_lens[b];
  const int npages = (L + P - 1) / P;
  const int ns = (npages + a.pps - 1) / a.pps;
  const float* ml = a.ws_ml + ((int64_t)u * a.nsplit * a.R + rr) * 2;
  const float* po = a.ws_o + ((int64_t)u * a.nsplit * a.R + rr) * D + E * lane;
  float M = NEG_INF;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[(int64_t)s * a.R * 2]);
  float l = 0.f, x[E];
#pragma unroll
  for (int i = 0; i < E; ++i) x[i] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float ms = ml[(int64_t)s * a.R * 2];
    if (ms == NEG_INF) continue;
    const float w = exp2f(ms - M);
    l += w * ml[(int64_t)s * a.R * 2 + 1];
    const float* os = po + (int64_t)s * a.R * D;
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] += w * os[i];
  }
  const float inv = l > 0.f ? a.v_out_scale / l : 0.f;
#pragma unroll
  for (int i = 0; i < E; ++i) x[i] *= inv;
  if constexpr (VROT) {
    fwht_wave<E>(x, lane);
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] *= 0.0625f;
  }
  const int qi = rr / a.G, qh = h * a.G + (rr - qi * a.G);
  const int64_t orow = ((int64_t)b * a.n_q + qi) * a.H_q + qh;
  float* op = a.out + orow * D + E * lane;
#pragma unroll
  for (int i = 0; i < E; ++i) op[i] = x[i];
  if (a.lse != nullptr && lane == 0) a.lse[orow] = l > 0.f ? (M + __log2f(l)) * 0.69314718055994531f : NEG_INF;
}

// ----------------------------------------------------------- launchers

template <int FMT, int D>
static hipError_t launch_split_t(const Geometry& geo, const DecodeArgs& a, hipStream_t stream) {
  const int units = a.B * geo.H_kv;
  const int tiles = (a.R + 15) / 16;
  hipLaunchKernelGGL((decode_split_kernel<FMT, D>), dim3((unsigned)a.nsplit * (unsigned)units, tiles), dim3(256), 0,
                     stream, geo, a);
  return hipGetLastError();
}

hipError_t launch_decode_split(const Geometry& geo, const DecodeArgs& a, hipStream_t stream) {
#define KVQ_SPLIT_CASE(F, DD) \
  if (geo.fmt == F && geo.D == DD) return launch_split_t<F, DD>(geo, a, stream);
  KVQ_SPLIT_CASE(F_BF16, 128) KVQ_SPLIT_CASE(F_BF16, 256)
  KVQ_SPLIT_CASE(F_FP8_ROW, 128) KVQ_SPLIT_CASE(F_FP8_ROW, 256)
  KVQ_SPLIT_CASE(F_FP8_TENSOR, 128) KVQ_SPLIT_CASE(F_FP8_TENSOR, 256)
  KVQ_SPLIT_CASE(F_MXFP8, 128) KVQ_SPLIT_CASE(F_MXFP8, 256)
  KVQ_SPLIT_CASE(F_INT8_G64, 256) KVQ_SPLIT_CASE(F_NVFP4_G16, 256) KVQ_SPLIT_CASE(F_K8V4, 256)
#undef KVQ_SPLIT_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const Geometry& geo, const DecodeArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * geo.H_kv * a.R;
  const unsigned blocks = (unsigned)((rows + 3) / 4);
  if (blocks == 0) return hipSuccess;
  const bool vrot = v_rotated(geo.fmt);
  if (geo.D == 256 && vrot)
    hipLaunchKernelGGL((decode_combine_kernel<256, true>), dim3(blocks), dim3(256), 0, stream, a, geo.P, geo.H_kv);
  else if (geo.D == 256)
    hipLaunchKernelGGL((decode_combine_kernel<256, false>), dim3(blocks), dim3(256), 0, stream, a, geo.P, geo.H_kv);
  else if (geo.D == 128 && !vrot)
    hipLaunchKernelGGL((decode_combine_kernel<128, false>), dim3(blocks), dim3(256), 0, stream, a, geo.P, geo.H_kv);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kvq
