// kvq_format.hpp -- format registry and page geometry (host and device).
//
// Formats (NInfer KV-cache quantization guide, section on the five formats;
// TokenSpeed article, --kv-cache-dtype section for mxfp8 and fp8_e4m3; Qwen
// FP8-KV article for the per-tensor symmetric FP8 scheme):
//
//   format       K codec        V codec        K rot  V rot
//   BF16         bf16 bits      fp16           no     no
//   INT8_G64     int8 / 64      int8 / 64      yes    no
//   FP8_ROW      e4m3 / row     e4m3 / row     no     no
//   NVFP4_G16    e2m1 / 16      e2m1 / 16      yes    yes
//   K8V4         e4m3 / row     e2m1 / 16      no     yes
//   MXFP8        e4m3 / 32      e4m3 / 32      no     no
//   FP8_TENSOR   e4m3 tensor    e4m3 tensor    no     no
//
// Page geometry.  A page holds H_kv head blocks; a head block is the four
// planes K codes | K scales | V codes | V scales, each padded to 128 bytes.
// Each plane is a run of P/16 token blocks (16 consecutive slots).  Inside
// a token block, with local token t in 0..15:
//
//   K codes, b bits per value, vpc = 128/b values per 16-byte chunk:
//     kk = d/32, g = (d%32)/8, e = d%8, i = kk/(vpc/8), j = (kk%(vpc/8))*8 + e
//     byte = i*1024 + (g*16 + t)*16 + j*b/8      (4-bit: j even -> low nibble)
//   This is the A-operand order of v_mfma_*_16x16x32: lane g*16+t holds
//   the 8 values k = 8g..8g+7 of k-step kk for token t, and one 16-byte load
//   per lane fetches vpc/8 consecutive k-steps.
//
//   V codes, t = 4g + e, d = 16*jt + n:
//     8-bit:  byte = (jt/4)*1024 + (g*16+n)*16 + (jt%4)*4 + e
//     16-bit: byte = (jt/2)*1024 + (g*16+n)*16 + (jt%2)*8 + 2e
//     4-bit:  byte = (jt/8)*1024 + (g*16+n)*16 + (jt%8)*2 + e/2,
//             high nibble for odd e (a byte holds column n of the token
//             pair 4g + 2p, 4g + 2p + 1)
//   This is the B-operand order of v_mfma_f32_16x16x16_f16 for the product
//   P (rows x tokens) . V (tokens x d): lane g*16+n holds tokens 4g..4g+3 of
//   column n of n-tile jt; for 4-bit codes each byte converts straight into
//   the f16 pair (4g + 2p, 4g + 2p + 1) of one operand register.
//
//   Scales, G groups per row: fp16 scales at (t*G + grp)*2; byte scales of
//   K planes and of 8-bit V planes at t*G + grp; byte scales of 4-bit V
//   planes (UE4M3, UE8M0) at (t/4)*4G + grp*4 + t%4.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define KVQ_HD __host__ __device__
#else
#define KVQ_HD
#endif

namespace kvq {

enum Codec : int {
  C_BF16 = 0,    // raw bf16 bits
  C_F16 = 1,     // IEEE fp16
  C_I8G64 = 2,   // int8, fp16 scale per 64
  C_E4ROW = 3,   // e4m3, fp16 scale per row
  C_E2G16 = 4,   // e2m1, ue4m3 scale per 16
  C_E4MX = 5,    // e4m3, ue8m0 scale per 32
  C_E4TEN = 6,   // e4m3, one fp32 scale per tensor (argument)
  C_E2MX = 7,    // e2m1, ue8m0 scale per 32
};

enum Format : int {
  F_BF16 = 0, F_INT8_G64 = 1, F_FP8_ROW = 2, F_NVFP4_G16 = 3, F_K8V4 = 4, F_MXFP8 = 5, F_FP8_TENSOR = 6,
  F_MXFP4 = 7, F_COUNT = 8
};

// Kernel variant tags (template arguments, never a descriptor's format):
// F_MXFP8 | VARIANT_QMX is the MXFP8 cache read with the query rounded to
// MXFP8 too and Q.K on the block-scaled fp8 matrix cores.  VARIANT_PACK
// (formats whose query goes to the matrix cores in two pieces: INT8-G64's
// two int8 digits, the f16 hi + lo of NVFP4 and MXFP4) is the kernel for at
// most 8 query rows per kv head, which puts both pieces into one 16-column
// operand (piece 1 in columns 0-7, piece 2 in columns 8-15) and so needs one
// Q.K product per k-step instead of two.  The format predicates below look
// at the format bits only.
constexpr int VARIANT_QMX = 0x100;
constexpr int VARIANT_PACK = 0x200;
KVQ_HD constexpr int base_format(int f) { return f & 0xFF; }

KVQ_HD constexpr int k_codec(int f) {
  f = base_format(f);
  return f == F_BF16 ? C_BF16 : f == F_INT8_G64 ? C_I8G64 : f == F_FP8_ROW ? C_E4ROW
       : f == F_NVFP4_G16 ? C_E2G16 : f == F_K8V4 ? C_E4ROW : f == F_MXFP8 ? C_E4MX : f == F_MXFP4 ? C_E2MX : C_E4TEN;
}
KVQ_HD constexpr int v_codec(int f) {
  f = base_format(f);
  return f == F_BF16 ? C_F16 : f == F_INT8_G64 ? C_I8G64 : f == F_FP8_ROW ? C_E4ROW
       : f == F_NVFP4_G16 ? C_E2G16 : f == F_K8V4 ? C_E2G16 : f == F_MXFP8 ? C_E4MX : f == F_MXFP4 ? C_E2MX : C_E4TEN;
}
KVQ_HD constexpr bool k_rotated(int f) {
  return base_format(f) == F_INT8_G64 || base_format(f) == F_NVFP4_G16 || base_format(f) == F_MXFP4;
}
KVQ_HD constexpr bool v_rotated(int f) {
  return base_format(f) == F_NVFP4_G16 || base_format(f) == F_K8V4 || base_format(f) == F_MXFP4;
}
// Planes with a per-tensor fp32 scale (the descriptor's k_scale / v_scale):
// FP8-tensor, and the two-level form of the NVFP4 planes (1 = single level).
KVQ_HD constexpr bool k_tensor_scaled(int f) {
  return base_format(f) == F_FP8_TENSOR || base_format(f) == F_NVFP4_G16;
}
KVQ_HD constexpr bool v_tensor_scaled(int f) {
  return base_format(f) == F_FP8_TENSOR || base_format(f) == F_NVFP4_G16 || base_format(f) == F_K8V4;
}

KVQ_HD constexpr int codec_bits(int c) { return (c == C_BF16 || c == C_F16) ? 16 : (c == C_E2G16 || c == C_E2MX) ? 4 : 8; }
// the scale is a power of two (UE8M0 byte): codes are scaled exactly by ldexp
KVQ_HD constexpr bool mx_scaled(int c) { return c == C_E4MX || c == C_E2MX; }
// group size along head_dim (0 = no per-row scales; -1 = whole row)
KVQ_HD constexpr int codec_group(int c) {
  return c == C_I8G64 ? 64 : c == C_E4ROW ? -1 : c == C_E2G16 ? 16 : (c == C_E4MX || c == C_E2MX) ? 32 : 0;
}
KVQ_HD constexpr int scale_bytes(int c) {
  return (c == C_I8G64 || c == C_E4ROW) ? 2 : (c == C_E2G16 || c == C_E4MX || c == C_E2MX) ? 1 : 0;
}
KVQ_HD constexpr int n_groups(int c, int D) {
  return codec_group(c) == 0 ? 0 : codec_group(c) < 0 ? 1 : D / codec_group(c);
}

constexpr int TOKEN_BLOCK = 16;
constexpr int PLANE_ALIGN = 128;

KVQ_HD constexpr int64_t pad_plane(int64_t n) { return (n + PLANE_ALIGN - 1) / PLANE_ALIGN * PLANE_ALIGN; }
KVQ_HD constexpr int code_block_bytes(int c, int D) { return TOKEN_BLOCK * D * codec_bits(c) / 8; }
KVQ_HD constexpr int scale_block_bytes(int c, int D) { return TOKEN_BLOCK * n_groups(c, D) * scale_bytes(c); }

// Byte offsets of the four planes inside a head block, and the sizes.
struct Geometry {
  int fmt, D, P, H_kv;
  int kc, vc;                 // codecs
  int kcode_blk, kscale_blk;  // per 16-token block
  int vcode_blk, vscale_blk;
  int64_t off_kc, off_ks, off_vc, off_vs;
  int64_t head_bytes, page_bytes;
};

KVQ_HD inline Geometry make_geometry(int fmt, int D, int P, int H_kv) {
  Geometry g{};
  g.fmt = fmt; g.D = D; g.P = P; g.H_kv = H_kv;
  g.kc = k_codec(fmt); g.vc = v_codec(fmt);
  g.kcode_blk = code_block_bytes(g.kc, D);
  g.kscale_blk = scale_block_bytes(g.kc, D);
  g.vcode_blk = code_block_bytes(g.vc, D);
  g.vscale_blk = scale_block_bytes(g.vc, D);
  const int nb = P / TOKEN_BLOCK;
  g.off_kc = 0;
  g.off_ks = g.off_kc + pad_plane((int64_t)nb * g.kcode_blk);
  g.off_vc = g.off_ks + pad_plane((int64_t)nb * g.kscale_blk);
  g.off_vs = g.off_vc + pad_plane((int64_t)nb * g.vcode_blk);
  g.head_bytes = g.off_vs + pad_plane((int64_t)nb * g.vscale_blk);
  g.page_bytes = g.head_bytes * H_kv;
  return g;
}

// In-block byte offset of K element (t, d) for a codec of `bits` bits.
KVQ_HD constexpr int k_code_byte(int bits, int t, int d) {
  // vpc/8 k-steps per chunk: 16-bit 1, 8-bit 2, 4-bit 4
  return ((d / 32) / (16 / bits)) * 1024 + ((((d % 32) / 8) * 16 + t) * 16)
         + ((((d / 32) % (16 / bits)) * 8 + (d % 8)) * bits) / 8;
}

// Is the format/head_dim/page_size combination supported?
KVQ_HD constexpr bool supported(int fmt, int D, int P) {
  return fmt >= 0 && fmt < F_COUNT && (P == 64 || P == 128) &&
         ((k_rotated(fmt) || v_rotated(fmt)) ? D == 256 : (D == 128 || D == 256));
}

}  // namespace kvq
