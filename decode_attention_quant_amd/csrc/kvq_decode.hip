// kvq_decode.hip -- split-K decode attention over the compressed paged cache.
//
// Every decode step reads all cached K/V of each sequence, so the bytes
// stored per token set the speed (NInfer KV-cache guide, section on why the
// cache is quantized; Qwen FP8-KV article, bandwidth section).  This kernel
// therefore streams each page plane exactly once with 16-byte loads and does
// the rest in registers.
//
// Schedule (stream-K): the 16-token blocks of every (sequence b, kv head h)
// unit, u = b * H_kv + h, form one flat range; workgroup x of the grid
// (x, row tile) takes an equal slice of it (at least 128 blocks), so every
// workgroup streams the same number of bytes whatever the length mix.  A
// unit wholly inside one slice is finished in place (normalized, V rotated
// back, lse written); a unit cut by slice ends leaves one partial (m, l, o)
// per slice for decode_combine_kernel.  The rows of a workgroup are the
// R = G * n_q query rows sharing one kv head (GQA group times MTP tokens,
// 16 per row tile).  Of its 4 waves, wave w takes blocks w, w + 4, ... and
// keeps its own online-softmax state; the waves merge through LDS.
//
// Per token block (one wave, 16 tokens x 16 rows):
//   S = K_blk . Q^T on the matrix cores, K codes expanded exactly:
//     BF16            bf16 K x bf16 q               (16x16x32 bf16)
//     FP8 row/tensor  E4M3 -> bf16 (exact) x bf16 q; row scale on S
//     MXFP8           E4M3 -> bf16 x bf16 q per 32-wide k-step, scaled by
//                     2^e of that group before summing
//     INT8-G64        int8 K x rotated q in two int8 digits (16x16x64 i8),
//                     group scale on each 64-wide integer partial sum
//     NVFP4 (K)       E2M1 x UE4M3 -> f16 (exact) x rotated q as f16 hi + lo
//   online softmax in base 2, masking t >= L and the MTP causal rule;
//   O (16 rows x D) += P . V_blk (16x16x16 f16), P rounded to f16 and V
//   expanded to f16 with its scale folded in: exact for fp16 V and for
//   E2M1 x UE4M3; one f16 rounding of code x scale for int8 and E4M3 with
//   an fp16 scale and for E4M3 x 2^e; the per-tensor V scale multiplies the
//   output instead.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kvq_device.hpp"
#include "kvq_encode.hpp"
#include "kvq_internal.hpp"

namespace kvq {

template <int FMT, int D>
struct DT {
  static constexpr int KC = k_codec(FMT), VC = v_codec(FMT);
  static constexpr int KBITS = codec_bits(KC), VBITS = codec_bits(VC);
  static constexpr bool QI8 = KC == C_I8G64;    // Q.K on the int8 matrix cores, q in two int8 pieces
  static constexpr bool QF16 = KC == C_E2G16;   // Q.K in f16, q split into f16 hi + lo
  static constexpr bool QROT = k_rotated(FMT);  // q is rotated first (K was)
  static constexpr bool VROT = v_rotated(FMT);
  static constexpr int KSTEPS = D / 32;
  static constexpr int QSTEPS = QI8 ? D / 64 : D / 32;  // MFMA k-steps of Q.K
  static constexpr int QPIECES = (QI8 || QF16) ? 2 : 1;
  // Bytes of one 16-token block in each plane, and their place in an LDS
  // stage (the four plane regions back to back).
  static constexpr int KB = code_block_bytes(KC, D), KSB = scale_block_bytes(KC, D);
  static constexpr int VB = code_block_bytes(VC, D), VSB = scale_block_bytes(VC, D);
  static constexpr int SK = 0, SKS = KB, SV = KB + KSB, SVS = KB + KSB + VB;
  static constexpr int STAGE = KB + KSB + VB + VSB;
  // Direct global->LDS loads (16 bytes per lane) that copy one block.
  static constexpr int NDMA = (KB + 1023) / 1024 + (KSB + 1023) / 1024 + (VB + 1023) / 1024 + (VSB + 1023) / 1024;
  // Blocks are staged through a per-wave ring of RING_S blocks in LDS,
  // RING_S - 1 of them in flight while one is consumed, where that fits in
  // RING_LDS bytes per workgroup (two workgroups per CU).  INT8-G64 keeps
  // its register pipeline: with q in two int8 pieces its loop is shorter
  // than the ring's extra LDS reads and waits cost (measured).
  static constexpr int RING_LDS = 72 * 1024;
  static constexpr int RING_FIT = RING_LDS / (4 * STAGE);
  static constexpr int RING_S = RING_FIT > 4 ? 4 : RING_FIT;
  static constexpr bool RING = RING_S >= 2 && FMT != F_INT8_G64;
  // Without the ring: Q operands in LDS (one ds_read_b128 per k-step) where
  // registers would otherwise spill.
  static constexpr bool QLDS = !RING;
  // Without the ring: prefetch whole blocks into a second register buffer
  // where it fits next to the O accumulators; otherwise reuse one buffer,
  // loading the next block's K as soon as Q.K is done and its V as soon as
  // P.V is done.
  static constexpr bool DOUBLE_BUF = D == 128 || FMT == F_FP8_ROW || FMT == F_FP8_TENSOR;
  static constexpr int NT = D / 16;
  static constexpr int KCH = D * KBITS / 512;                       // 16-B K chunks per lane per block
  static constexpr int VCH = VBITS * NT / 32;                       // 16-B V chunks per lane per block
  static constexpr int KSW = KC == C_E4ROW ? 2 : KC == C_I8G64 ? 8 : KC == C_E4MX ? D / 32 : KC == C_E2G16 ? 4 : 0;
  static constexpr int VSW = VC == C_E4ROW ? 2 : VC == C_I8G64 ? 8 : VC == C_E4MX ? D / 32 : VC == C_E2G16 ? 16 : 0;
  static constexpr int G = n_groups(KC, D) > 0 ? n_groups(KC, D) : 1;
};

// Tables the kernel only reads (page table, sequence lengths) are read
// through the constant address space, so uniform indexes become scalar
// loads: a vector load here would be counted by vmcnt, and waiting for it
// would also wait for every block prefetch issued before it.
typedef const __attribute__((address_space(4))) int32_t cint32;
__device__ __forceinline__ const cint32* as_const(const int32_t* p) { return (const cint32*)p; }

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

// Addresses of token block j (absolute block index within the unit).
struct BlockAddr {
  const uint8_t* hb;  // head block of the page holding block j
  int bip;            // block index inside the page
};
__device__ __forceinline__ BlockAddr block_addr(const uint8_t* head0, const Geometry& geo, const cint32* bt_row,
                                                int j) {
  const int bpp_log2 = geo.P == 128 ? 3 : 2;  // 16-token blocks per page: 8 or 4
  const int page = __builtin_amdgcn_readfirstlane(j >> bpp_log2);
  BlockAddr r;
  r.bip = j & ((1 << bpp_log2) - 1);
  r.hb = head0 + (int64_t)bt_row[page] * geo.page_bytes;
  return r;
}

// Load the K codes (and K scales) of token block j into registers.
template <int FMT, int D>
__device__ __forceinline__ void load_k(Buf<FMT, D>& buf, const uint8_t* head0, const Geometry& geo,
                                       const cint32* bt_row, int j, int lane) {
  using T = DT<FMT, D>;
  const BlockAddr ba = block_addr(head0, geo, bt_row, j);
  const int g = lane >> 4, c16 = lane & 15;
  const uint8_t* kc = ba.hb + geo.off_kc + (int64_t)ba.bip * geo.kcode_blk;
#pragma unroll
  for (int i = 0; i < T::KCH; ++i) buf.k[i] = *reinterpret_cast<const uint4*>(kc + i * 1024 + lane * 16);
  if constexpr (T::KSW > 0) {
    const uint8_t* ks = ba.hb + geo.off_ks + (int64_t)ba.bip * geo.kscale_blk;
    const int off = T::KC == C_E2G16 ? c16 * 16 : g * (4 * T::KSW);
    load_words(buf.ks, ks + off);
  }
}

// Load the V codes (and V scales) of token block j into registers.
template <int FMT, int D>
__device__ __forceinline__ void load_v(Buf<FMT, D>& buf, const uint8_t* head0, const Geometry& geo,
                                       const cint32* bt_row, int j, int lane) {
  using T = DT<FMT, D>;
  const BlockAddr ba = block_addr(head0, geo, bt_row, j);
  const int g = lane >> 4;
  const uint8_t* vc = ba.hb + geo.off_vc + (int64_t)ba.bip * geo.vcode_blk;
#pragma unroll
  for (int q = 0; q < T::VCH; ++q) buf.v[q] = *reinterpret_cast<const uint4*>(vc + q * 1024 + lane * 16);
  if constexpr (T::VSW > 0) {
    const uint8_t* vs = ba.hb + geo.off_vs + (int64_t)ba.bip * geo.vscale_blk;
    load_words(buf.vs, vs + g * (4 * T::VSW));
  }
}

template <int FMT, int D>
__device__ __forceinline__ void load_block(Buf<FMT, D>& buf, const uint8_t* head0, const Geometry& geo,
                                           const cint32* bt_row, int j, int lane) {
  load_k<FMT, D>(buf, head0, geo, bt_row, j, lane);
  load_v<FMT, D>(buf, head0, geo, bt_row, j, lane);
}

// ----------------------------------------------------------- LDS ring
// A wave copies each 16-token block into a stage of its own LDS ring with
// direct global->LDS loads (global_load_lds_dwordx4: lane l's 16 bytes land
// at the stage address + 16 l), which hold no registers while in flight.
// Completion is tracked with explicit vmcnt waits: inside the block loop
// these copies are the only vector-memory instructions, and they complete in
// order.  Stages are read back with ds_read_b128 in inline asm that waits for
// its own results, so the compiler's conservative wait for every
// outstanding copy before an LDS read never enters the loop.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

template <int BYTES>
__device__ __forceinline__ void copy_plane(uint32_t dst, const uint8_t* src, int lane) {
#pragma unroll
  for (int c = 0; c < BYTES / 1024; ++c)
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(src + c * 1024 + lane * 16),
                                     (lds_void_t*)(uintptr_t)(dst + c * 1024), 16, 0, 0);
  constexpr int REM = BYTES % 1024;
  if constexpr (REM > 0) {
    if (lane < REM / 16)
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(src + (BYTES / 1024) * 1024 + lane * 16),
                                       (lds_void_t*)(uintptr_t)(dst + (BYTES / 1024) * 1024), 16, 0, 0);
  }
}

// Start copying token block j into the stage at LDS byte address `stage`.
template <int FMT, int D>
__device__ __forceinline__ void stage_block(uint32_t stage, const uint8_t* head0, const Geometry& geo,
                                            const cint32* bt_row, int j, int lane) {
  using T = DT<FMT, D>;
  const BlockAddr ba = block_addr(head0, geo, bt_row, j);
  copy_plane<T::KB>(stage + T::SK, ba.hb + geo.off_kc + (int64_t)ba.bip * T::KB, lane);
  if constexpr (T::KSB > 0) copy_plane<T::KSB>(stage + T::SKS, ba.hb + geo.off_ks + (int64_t)ba.bip * T::KSB, lane);
  copy_plane<T::VB>(stage + T::SV, ba.hb + geo.off_vc + (int64_t)ba.bip * T::VB, lane);
  if constexpr (T::VSB > 0) copy_plane<T::VSB>(stage + T::SVS, ba.hb + geo.off_vs + (int64_t)ba.bip * T::VSB, lane);
}

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt fields at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until every copy of a block is done when `after` blocks (wave-
// uniform, < S) were staged behind it.
template <int NDMA, int S>
__device__ __forceinline__ void wait_staged(int after) {
  if constexpr (S > 3) {
    if (after >= 3) { wait_vmcnt<3 * NDMA>(); return; }
  }
  if constexpr (S > 2) {
    if (after >= 2) { wait_vmcnt<2 * NDMA>(); return; }
  }
  if (after >= 1) { wait_vmcnt<NDMA>(); return; }
  wait_vmcnt<0>();
}

// NC 16-byte code chunks at c + i * CS (i < NC) and SW scale words at s
// (consecutive), read from LDS in one asm block that waits for them.
template <int NC, int CS, int SW>
__device__ __forceinline__ void lds_read_part(uint4 (&c)[NC], uint32_t (&w)[SW > 0 ? SW : 1], uint32_t ca,
                                              uint32_t sa) {
  static_assert(NC == 2 || NC == 4, "");
  static_assert(SW == 0 || SW == 2 || SW == 4 || SW == 8 || SW == 16, "");
#define KVQ_R(o, a, off) "ds_read_b128 %" #o ", %" #a " offset:%" #off "\n\t"
#define KVQ_W "s_waitcnt lgkmcnt(0)"
  if constexpr (NC == 2) {
    if constexpr (SW == 0) {
      asm volatile(KVQ_R(0, 2, 3) KVQ_R(1, 2, 4) KVQ_W
                   : "=&v"(c[0]), "=&v"(c[1]) : "v"(ca), "i"(0), "i"(CS) : "memory");
    } else if constexpr (SW == 2) {
      uint2 s0;
      asm volatile(KVQ_R(0, 3, 5) KVQ_R(1, 3, 6) "ds_read_b64 %2, %4\n\t" KVQ_W
                   : "=&v"(c[0]), "=&v"(c[1]), "=&v"(s0) : "v"(ca), "v"(sa), "i"(0), "i"(CS) : "memory");
      w[0] = s0.x; w[1] = s0.y;
    } else if constexpr (SW == 4) {
      uint4 s0;
      asm volatile(KVQ_R(0, 3, 5) KVQ_R(1, 3, 6) KVQ_R(2, 4, 5) KVQ_W
                   : "=&v"(c[0]), "=&v"(c[1]), "=&v"(s0) : "v"(ca), "v"(sa), "i"(0), "i"(CS) : "memory");
      w[0] = s0.x; w[1] = s0.y; w[2] = s0.z; w[3] = s0.w;
    } else if constexpr (SW == 8) {
      uint4 s0, s1;
      asm volatile(KVQ_R(0, 4, 6) KVQ_R(1, 4, 7) KVQ_R(2, 5, 6) KVQ_R(3, 5, 8) KVQ_W
                   : "=&v"(c[0]), "=&v"(c[1]), "=&v"(s0), "=&v"(s1) : "v"(ca), "v"(sa), "i"(0), "i"(CS), "i"(16)
                   : "memory");
      w[0] = s0.x; w[1] = s0.y; w[2] = s0.z; w[3] = s0.w; w[4] = s1.x; w[5] = s1.y; w[6] = s1.z; w[7] = s1.w;
    } else {
      uint4 s0, s1, s2, s3;
      asm volatile(KVQ_R(0, 6, 8) KVQ_R(1, 6, 9) KVQ_R(2, 7, 8) KVQ_R(3, 7, 10) KVQ_R(4, 7, 11) KVQ_R(5, 7, 12) KVQ_W
                   : "=&v"(c[0]), "=&v"(c[1]), "=&v"(s0), "=&v"(s1), "=&v"(s2), "=&v"(s3)
                   : "v"(ca), "v"(sa), "i"(0), "i"(CS), "i"(16), "i"(32), "i"(48) : "memory");
      const uint4 ss[4] = {s0, s1, s2, s3};
#pragma unroll
      for (int i = 0; i < 4; ++i) { w[4 * i] = ss[i].x; w[4 * i + 1] = ss[i].y; w[4 * i + 2] = ss[i].z; w[4 * i + 3] = ss[i].w; }
    }
  } else {
    if constexpr (SW == 0) {
      asm volatile(KVQ_R(0, 4, 5) KVQ_R(1, 4, 6) KVQ_R(2, 4, 7) KVQ_R(3, 4, 8) KVQ_W
                   : "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3])
                   : "v"(ca), "i"(0), "i"(CS), "i"(2 * CS), "i"(3 * CS) : "memory");
    } else if constexpr (SW == 2) {
      uint2 s0;
      asm volatile(KVQ_R(0, 5, 7) KVQ_R(1, 5, 8) KVQ_R(2, 5, 9) KVQ_R(3, 5, 10) "ds_read_b64 %4, %6\n\t" KVQ_W
                   : "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3]), "=&v"(s0)
                   : "v"(ca), "v"(sa), "i"(0), "i"(CS), "i"(2 * CS), "i"(3 * CS) : "memory");
      w[0] = s0.x; w[1] = s0.y;
    } else if constexpr (SW == 4) {
      uint4 s0;
      asm volatile(KVQ_R(0, 5, 7) KVQ_R(1, 5, 8) KVQ_R(2, 5, 9) KVQ_R(3, 5, 10) KVQ_R(4, 6, 7) KVQ_W
                   : "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3]), "=&v"(s0)
                   : "v"(ca), "v"(sa), "i"(0), "i"(CS), "i"(2 * CS), "i"(3 * CS) : "memory");
      w[0] = s0.x; w[1] = s0.y; w[2] = s0.z; w[3] = s0.w;
    } else if constexpr (SW == 8) {
      uint4 s0, s1;
      asm volatile(KVQ_R(0, 6, 8) KVQ_R(1, 6, 9) KVQ_R(2, 6, 10) KVQ_R(3, 6, 11) KVQ_R(4, 7, 8) KVQ_R(5, 7, 12) KVQ_W
                   : "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3]), "=&v"(s0), "=&v"(s1)
                   : "v"(ca), "v"(sa), "i"(0), "i"(CS), "i"(2 * CS), "i"(3 * CS), "i"(16) : "memory");
      w[0] = s0.x; w[1] = s0.y; w[2] = s0.z; w[3] = s0.w; w[4] = s1.x; w[5] = s1.y; w[6] = s1.z; w[7] = s1.w;
    } else {
      uint4 s0, s1, s2, s3;
      asm volatile(KVQ_R(0, 8, 10) KVQ_R(1, 8, 11) KVQ_R(2, 8, 12) KVQ_R(3, 8, 13)
                   KVQ_R(4, 9, 10) KVQ_R(5, 9, 14) KVQ_R(6, 9, 15) KVQ_R(7, 9, 16) KVQ_W
                   : "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3]), "=&v"(s0), "=&v"(s1), "=&v"(s2), "=&v"(s3)
                   : "v"(ca), "v"(sa), "i"(0), "i"(CS), "i"(2 * CS), "i"(3 * CS), "i"(16), "i"(32), "i"(48)
                   : "memory");
      const uint4 ss[4] = {s0, s1, s2, s3};
#pragma unroll
      for (int i = 0; i < 4; ++i) { w[4 * i] = ss[i].x; w[4 * i + 1] = ss[i].y; w[4 * i + 2] = ss[i].z; w[4 * i + 3] = ss[i].w; }
    }
  }
#undef KVQ_R
#undef KVQ_W
}

// The K codes and scales of the block in `stage`, in the registers and lane
// order load_k would give.
template <int FMT, int D>
__device__ __forceinline__ void read_stage_k(Buf<FMT, D>& buf, uint32_t stage, int lane) {
  using T = DT<FMT, D>;
  const int g = lane >> 4, c16 = lane & 15;
  const uint32_t sa = stage + T::SKS + (T::KC == C_E2G16 ? c16 * 16 : g * (4 * T::KSW));
  lds_read_part<T::KCH, 1024, T::KSW>(buf.k, buf.ks, stage + T::SK + lane * 16, sa);
}

// The V codes and scales of the block in `stage`, as load_v would give them.
template <int FMT, int D>
__device__ __forceinline__ void read_stage_v(Buf<FMT, D>& buf, uint32_t stage, int lane) {
  using T = DT<FMT, D>;
  const int g = lane >> 4;
  lds_read_part<T::VCH, 1024, T::VSW>(buf.v, buf.vs, stage + T::SV + lane * 16, stage + T::SVS + g * (4 * T::VSW));
}

// ----------------------------------------------------------- operand expanders

// 8 E4M3 codes (two dwords) -> bf16x8, exact
__device__ __forceinline__ bf16x8 e4m3x8_bf16(uint32_t w0, uint32_t w1) {
  uint4 r;
  r.x = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, false));
  r.y = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, true));
  r.z = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, false));
  r.w = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, true));
  return bitcast<bf16x8>(r);
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
  return bitcast<f16x8>(make_uint4(bitcast<uint32_t>(a), bitcast<uint32_t>(b), bitcast<uint32_t>(c),
                                   bitcast<uint32_t>(d)));
}

// 8 E2M1 codes (one dword, element e in nibble e) -> f16x8, exact
__device__ __forceinline__ f16x8 e2m1x8_f16(uint32_t w) {
  uint4 r;
  r.x = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0));
  r.y = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1));
  r.z = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2));
  r.w = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3));
  return bitcast<f16x8>(r);
}

__device__ __forceinline__ uint32_t word(const uint4& q, int i) {
  return i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w;
}

// ----------------------------------------------------------- Q operands

template <int FMT, int D>
struct QOps {
  // B operands of S = K . Q^T, k-step kk, piece p (bf16 q; f16 hi, lo; or
  // int8 coarse, fine), as raw 16-byte lane values
  using T = DT<FMT, D>;
  uint4 reg[T::QLDS ? 1 : T::QSTEPS * T::QPIECES];
  const uint4* lds;
  int lane;
  __device__ __forceinline__ uint4 get(int kk, int p) const {
    if constexpr (T::QLDS) return lds[(kk * T::QPIECES + p) * 64 + lane];
    else return reg[kk * T::QPIECES + p];
  }
};

// ----------------------------------------------------------- S = K . Q^T

template <int FMT, int D>
__device__ __forceinline__ f32x4 qk_block(const Buf<FMT, D>& buf, const QOps<FMT, D>& qo, int lane) {
  using T = DT<FMT, D>;
  f32x4 S = {0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  if constexpr (T::KC == C_BF16) {
    // two independent accumulator chains (even / odd k-steps)
    f32x4 S1 = zero;
#pragma unroll
    for (int kk = 0; kk < T::KSTEPS; kk += 2) {
      S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(buf.k[kk]), bitcast<bf16x8>(qo.get(kk, 0)), S, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(buf.k[kk + 1]), bitcast<bf16x8>(qo.get(kk + 1, 0)), S1,
                                                   0, 0, 0);
    }
    S += S1;
  } else if constexpr (T::KC == C_E4ROW || T::KC == C_E4TEN) {
    f32x4 S1 = zero;
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) {
      S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_bf16(buf.k[i].x, buf.k[i].y), bitcast<bf16x8>(qo.get(2 * i, 0)), S, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_bf16(buf.k[i].z, buf.k[i].w), bitcast<bf16x8>(qo.get(2 * i + 1, 0)), S1, 0, 0, 0);
    }
    S += S1;
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
            e4m3x8_bf16(hh ? buf.k[i].z : buf.k[i].x, hh ? buf.k[i].w : buf.k[i].y), bitcast<bf16x8>(qo.get(kk, 0)),
            zero, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int bi = e * G + kk;  // token 4g+e, group kk
          const int ex = (int)((buf.ks[bi >> 2] >> (8 * (bi & 3))) & 0xFFu) - 127;
          S[e] += ldexpf(acc[e], ex);
        }
      }
    }
  } else if constexpr (T::KC == C_I8G64) {
    // one fp16 scale per 64 values = one 16-byte chunk = one int8 k-step:
    // the raw codes are the A operand; q = coarse + fine / 254 (int8 each)
    const i32x4 izero = {0, 0, 0, 0};
#pragma unroll
    for (int grp = 0; grp < T::KCH; ++grp) {
      const i32x4 kc = bitcast<i32x4>(buf.k[grp]);
      const i32x4 a1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(kc, bitcast<i32x4>(qo.get(grp, 0)), izero, 0, 0, 0);
      const i32x4 a2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(kc, bitcast<i32x4>(qo.get(grp, 1)), izero, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int hw = e * 4 + grp;  // halfword of token 4g+e, group grp
        const float sc = f16_bits_to_f32((buf.ks[hw >> 1] >> (16 * (hw & 1))) & 0xFFFFu);
        S[e] += (float)(a1[e] * 254 + a2[e]) * sc;  // |a1| <= 64*127*127: no int32 overflow
      }
    }
  } else if constexpr (T::KC == C_E2G16) {
    // E2M1 x UE4M3 is exact in f16: fold the group scale into the operand.
    // lane (g, t): k-step kk covers d in [32kk + 8g, +8) -> group 2kk + g/2
    const int gb = (lane >> 5) & 1;
    f32x4 Slo = zero;
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
        // hi and lo parts of q in separate chains
        S = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bitcast<f16x8>(qo.get(kk, 0)), S, 0, 0, 0);
        Slo = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bitcast<f16x8>(qo.get(kk, 1)), Slo, 0, 0, 0);
      }
    }
    S += Slo;
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
  } else {  // C_E2G16: bytes 2 (nt & 1) and 2 (nt & 1) + 1 of word (nt & 7) / 2 of chunk nt / 8
            // hold tokens (4g, 4g + 1) and (4g + 2, 4g + 3) of column n, the earlier token low
    const uint32_t w = word(buf.v[nt >> 3], (nt & 7) >> 1);
    f16x2 a, b;
    if (nt & 1) {
      a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
      b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
    } else {
      a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
      b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    }
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

// Maximum over the four lanes 16 g + c (g = 0..3) that share c, without an
// LDS round trip: each swap leaves x of this lane and of its partner at
// distance 16 (then 32) in the two results.
__device__ __forceinline__ float max_over_g(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(bitcast<uint32_t>(x), bitcast<uint32_t>(x), false, false);
  x = fmaxf(bitcast<float>((uint32_t)a[0]), bitcast<float>((uint32_t)a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(bitcast<uint32_t>(x), bitcast<uint32_t>(x), false, false);
  return fmaxf(bitcast<float>((uint32_t)b[0]), bitcast<float>((uint32_t)b[1]));
}

// Slack of the running maximum, in log2 units (see pv_phase).
constexpr float RESCALE_SLACK = 8.0f;

// 2^x with the hardware exp: results below 2^-126 flush to zero, which only
// drops probabilities far below anything that can change an fp32 sum
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ----------------------------------------------------------- tail blocks

// Zero the V codes and V scales of this lane's tokens 4g+e at or past
// `nvalid` (slots past the sequence end may hold any bytes, NaN codes
// included), so that tokens with zero probability add exactly zero.
template <int FMT, int D>
__device__ __forceinline__ void clear_tail(Buf<FMT, D>& buf, int nvalid, int g) {
  using T = DT<FMT, D>;
  const int nv = nvalid - 4 * g;  // valid tokens among this lane's four
  uint32_t bmask = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) bmask |= (e < nv) ? (0xFFu << (8 * e)) : 0u;
  const uint32_t h01 = (nv > 0 ? 0xFFFFu : 0u) | (nv > 1 ? 0xFFFF0000u : 0u);
  const uint32_t h23 = (nv > 2 ? 0xFFFFu : 0u) | (nv > 3 ? 0xFFFF0000u : 0u);
  // 4-bit codes: nibble i of every word belongs to token i % 4
  const uint32_t n16 = nv >= 4 ? 0xFFFFu : nv <= 0 ? 0u : (1u << (4 * nv)) - 1u;
  const uint32_t nmask = n16 | (n16 << 16);
#pragma unroll
  for (int q = 0; q < T::VCH; ++q) {
    if constexpr (T::VBITS == 16) {
      buf.v[q].x &= h01; buf.v[q].y &= h23; buf.v[q].z &= h01; buf.v[q].w &= h23;
    } else {
      const uint32_t m = T::VBITS == 4 ? nmask : bmask;
      buf.v[q].x &= m; buf.v[q].y &= m; buf.v[q].z &= m; buf.v[q].w &= m;
    }
  }
  if constexpr (T::VC == C_E4ROW) {
    buf.vs[0] &= h01;
    buf.vs[1] &= h23;
  } else if constexpr (T::VC == C_I8G64) {  // token e: words 2e, 2e+1
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e >= nv) { buf.vs[2 * e] = 0u; buf.vs[2 * e + 1] = 0u; }
  } else if constexpr (T::VC == C_E4MX) {  // token e: D/128 words
    constexpr int WPT = D / 128;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int w = 0; w < WPT; ++w)
        if (e >= nv) buf.vs[e * WPT + w] = 0u;
  } else if constexpr (T::VC == C_E2G16) {
#pragma unroll
    for (int w = 0; w < T::VSW; ++w) buf.vs[w] &= bmask;
  }
}

// ----------------------------------------------------------- fused append

// Encode and store the new tokens of sequence b, kv head h at positions
// [plo, phi) (all inside this workgroup's blocks): wave 0 the K rows (a
// quad per token), wave 1 the V rows (a row of 16 lanes per 4 tokens), with
// the write path's own encoders, so the bytes are those quantize-append
// stores.  Input token i of sequence b is row b * n_q + i of k_new / v_new.
template <int FMT, int D>
__device__ __forceinline__ void append_new_tokens(const DecodeArgs& a, const Geometry& geo, int b, int h, int L,
                                               int plo, int phi, int wave, int lane) {
  const int pnew = L - a.n_q;          // position of new token 0
  const int64_t tok0 = (int64_t)b * a.n_q;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  auto slot_of = [&](int64_t tok) -> int {
    const int p = pnew + (int)(tok - tok0);
    return p >= 0 ? bt[p / geo.P] * geo.P + p % geo.P : -1;
  };
  const int ilo = plo - pnew, ihi = phi - pnew;  // new-token indexes written here
  if (wave == 0) {
    const int q = lane & 3;
    for (int i0 = ilo; i0 < ihi; i0 += 16) {
      const int i = i0 + (lane >> 2);  // a whole quad shares it
      if (i < ihi) {
        const int64_t tok = tok0 + i;
        uint32_t raw[D / 8];
        enc::load_k_row<D>(raw, a.k_new + (tok * geo.H_kv + h) * D + q * (D / 4));
        enc::encode_k_row<FMT, D>(a.pool_w, raw, slot_of(tok), geo, h, a.enc_k_scale, q);
      }
    }
  } else if (wave == 1) {
    for (int i0 = ilo; i0 < ihi; i0 += 16)
      enc::v_row_group<FMT, D>(a.pool_w, a.v_new, slot_of, geo, a.enc_v_scale, h, lane & 15,
                               tok0 + i0 + 4 * (lane >> 4), tok0 + ilo, tok0 + ihi);
  }
}

// ----------------------------------------------------------- the kernel

// Blocks per split workgroup: an equal share of the T blocks, but at least
// ceil(T / 256) clamped to [16, 128], so that when the sequences are shorter
// than the grid was sized for, about 256 workgroups (one per CU) get longer
// ranges and the rest find theirs empty, instead of every range shrinking
// to a few blocks that each leave a partial result.
__host__ __device__ __forceinline__ int blocks_per_workgroup(int total, int nwg) {
  const int per = (total + nwg - 1) / nwg;
  int lo = (total + 255) / 256;
  lo = lo < 16 ? 16 : (lo > 128 ? 128 : lo);
  return per > lo ? per : lo;
}

// LDS layout of the split kernel: prefix table int [B + 1] (rounded to 16),
// m and l float [4][16] each, 16 spare floats (q maxima), the Q operand
// store when it lives in LDS, then one area that holds the 4 waves' block
// rings during the block loop and the merge area float [4][Rt][D] after it.
template <int FMT, int D>
__host__ __device__ constexpr size_t split_lds_bytes(int B, int R) {
  using T = DT<FMT, D>;
  const int rt = R < 16 ? R : 16;
  const size_t cum = (size_t)((B + 1 + 15) / 16 * 16);
  const size_t merge = 4 * (size_t)rt * D * sizeof(float);
  const size_t ring = T::RING ? (size_t)4 * T::RING_S * T::STAGE : 0;
  return (cum + 64 + 64 + 16) * sizeof(float) + (T::QLDS ? (size_t)T::QSTEPS * T::QPIECES * 64 * 16 : 0) +
         (merge > ring ? merge : ring);
}

// FUSED: also store the new tokens first (DecodeArgs::pool_w); a separate
// instantiation, so the encoders' registers never weigh on the plain kernel.
template <int FMT, int D, bool FUSED>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(Geometry geo, DecodeArgs a) {
  using T = DT<FMT, D>;
  constexpr float NEG_INF = -__builtin_inff();
  extern __shared__ float lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int w = blockIdx.x, rt = blockIdx.y;
  const int Rt = min(16, a.R - 16 * rt);
  int* cum = reinterpret_cast<int*>(lds);
  float* sm_m = lds + (a.B + 1 + 15) / 16 * 16;
  float* sm_l = sm_m + 64;
  float* qexp = sm_l + 64;
  uint4* qst = reinterpret_cast<uint4*>(qexp + 16);
  float* sm_o = reinterpret_cast<float*>(qst + (T::QLDS ? T::QSTEPS * T::QPIECES * 64 : 0));
  // LDS byte address of this wave's ring (the low 32 bits of a generic
  // pointer into LDS are its LDS offset)
  const uint32_t ring0 = (uint32_t)(uintptr_t)(void*)sm_o + (uint32_t)(wave * T::RING_S * T::STAGE);

  // ---- cum[b] = H_kv * sum_{b' < b} ceil(L_b' / 16): the flat block index
  //      of unit (b, 0).  Each thread scans a contiguous run, then the runs'
  //      totals are scanned by wave 0.
  {
    const int per_t = (a.B + 255) / 256;
    const int b0 = threadIdx.x * per_t;
    int run = 0;
    for (int i = 0; i < per_t; ++i) {
      const int bb = b0 + i;
      if (bb < a.B) run += ((a.seq_lens[bb] + 15) >> 4) * geo.H_kv;
    }
    float* tot = sm_o;  // scratch [257] before the merge area is used (it holds >= 512)
    tot[threadIdx.x] = __int_as_float(run);
    __syncthreads();
    if (threadIdx.x < 64) {
      int v[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[i] = __float_as_int(tot[4 * threadIdx.x + i]); sum += v[i]; }
      int incl = sum;  // inclusive scan of the lane sums
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const int t = __shfl_up(incl, m);
        if ((int)threadIdx.x >= m) incl += t;
      }
      int ex = incl - sum;
#pragma unroll
      for (int i = 0; i < 4; ++i) { tot[4 * threadIdx.x + i] = __int_as_float(ex); ex += v[i]; }
      if (threadIdx.x == 63) tot[256] = __int_as_float(ex);  // grand total
    }
    __syncthreads();
    int base = __float_as_int(tot[threadIdx.x]);
    for (int i = 0; i < per_t; ++i) {
      const int bb = b0 + i;
      if (bb < a.B) {
        cum[bb] = base;
        base += ((a.seq_lens[bb] + 15) >> 4) * geo.H_kv;
      }
    }
    if (threadIdx.x == 0) cum[a.B] = __float_as_int(tot[256]);
    __syncthreads();
  }
  const int total = cum[a.B];
  if (w == 0 && rt == 0)
    for (int i = threadIdx.x; i <= a.B; i += 256) a.ws_cum[i] = cum[i];
  const int per = blocks_per_workgroup(total, a.nwg);
  int x = w * per;
  const int x_end = min(total, x + per);

  while (x < x_end) {
    // ---- the unit that holds flat block x: b = last index with cum[b] <= x
    int lo = 0, hi = a.B;  // cum[lo] <= x < cum[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cum[mid] <= x) lo = mid; else hi = mid;
    }
    const int b = __builtin_amdgcn_readfirstlane(lo);
    const int L = as_const(a.seq_lens)[b];
    const int nb = (L + 15) >> 4;
    const int within = x - cum[b];
    const int h = __builtin_amdgcn_readfirstlane(within / nb);
    const int blk0 = __builtin_amdgcn_readfirstlane(within - h * nb);
    const int seg_end = min(x_end, cum[b] + (h + 1) * nb);
    const int nblk = __builtin_amdgcn_readfirstlane(seg_end - x);
    const bool whole = blk0 == 0 && nblk == nb;
    const int u = b * geo.H_kv + h;

    // ---- fused step: store the new tokens that fall in this segment's
    //      blocks before any of those blocks is staged.  No other workgroup
    //      reads them (one row tile), and this one reads them through the
    //      same L2, so it is enough that its stores and atomics have
    //      completed (vmcnt 0) before the barrier: a workgroup-scope fence,
    //      not a device-wide L2 write-back.  The atomics of 4-bit V codes
    //      touch only cache lines of this block's own code plane.
    if constexpr (FUSED) {
      const int plo = max(max(L - a.n_q, 0), 16 * blk0), phi = min(L, 16 * (blk0 + nblk));
      if (plo < phi) {
        append_new_tokens<FMT, D>(a, geo, b, h, L, plo, phi, wave, lane);
        wait_vmcnt<0>();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      }
    }

    // ---- query rows of this tile: row r (= c16 in S layout) -> (i, head)
    const int r = c16;
    const int rr = 16 * rt + r;
    const bool row_ok = r < Rt;
    const int qi = rr / a.G, qh = h * a.G + (rr - qi * a.G);
    const int limit = row_ok ? L - a.n_q + qi : -1;  // last visible position of this row
    float crow = a.qk_scale;

    QOps<FMT, D> qo;
    qo.lane = lane;
    qo.lds = qst;
    uint4 qv[T::QSTEPS * T::QPIECES];
    if constexpr (!T::QROT) {
      const uint16_t* qp = a.q + (((int64_t)b * a.n_q + qi) * a.H_q + qh) * D;
#pragma unroll
      for (int kk = 0; kk < T::QSTEPS; ++kk) {
        uint4 q4 = make_uint4(0, 0, 0, 0);
        if (row_ok) q4 = *reinterpret_cast<const uint4*>(qp + 32 * kk + 8 * g);
        qv[kk] = q4;
      }
    } else {
      // q' = H q / 16 in fp32 (rows spread over the waves, through LDS)
      float* qrot = sm_o;  // [Rt][D]
      constexpr int E = D / 64;
      for (int row = wave; row < Rt; row += 4) {
        const int rr2 = 16 * rt + row;
        const int i2 = rr2 / a.G, h2 = h * a.G + (rr2 - i2 * a.G);
        const uint16_t* qp = a.q + (((int64_t)b * a.n_q + i2) * a.H_q + h2) * D + E * lane;
        float xq[E];
        const uint2 q2 = *reinterpret_cast<const uint2*>(qp);
        xq[0] = bf16_to_f32(q2.x & 0xFFFFu); xq[1] = bf16_to_f32(q2.x >> 16);
        xq[2] = bf16_to_f32(q2.y & 0xFFFFu); xq[3] = bf16_to_f32(q2.y >> 16);
        fwht_wave<E>(xq, lane);
        float am = 0.f;
#pragma unroll
        for (int i = 0; i < E; ++i) { xq[i] *= 0.0625f; am = fmaxf(am, fabsf(xq[i])); }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) am = fmaxf(am, __shfl_xor(am, m));
#pragma unroll
        for (int i = 0; i < E; ++i) qrot[row * D + E * lane + i] = xq[i];
        if (lane == 0) qexp[row] = am;
      }
      __syncthreads();
      const float am = row_ok ? qexp[r] : 0.f;
      if constexpr (T::QI8) {
        // q' ~ (c1 + c2 / 254) / inv, int8 c1 = RN(q' inv), c2 = RN(254 (q' inv - c1)),
        // inv = 127 / max|q'|: error below max|q'| / 64516 per element
        const float inv = am > 0.f ? 127.0f / am : 0.f;
        crow = am > 0.f ? a.qk_scale * (am / (127.0f * 254.0f)) : 0.f;
#pragma unroll
        for (int kk = 0; kk < T::QSTEPS; ++kk) {
          uint32_t w1[4] = {0, 0, 0, 0}, w2[4] = {0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            // k-slot 16g + j of int8 k-step kk <-> d as laid out in the K chunk
            const int d = 64 * kk + (j < 8 ? 8 * g + j : 32 + 8 * g + (j - 8));
            const float v = row_ok ? qrot[r * D + d] * inv : 0.f;
            const float c1 = fmaxf(fminf(rintf(v), 127.f), -127.f);
            const float c2 = fmaxf(fminf(rintf((v - c1) * 254.0f), 127.f), -127.f);
            w1[j >> 2] |= ((uint32_t)(int)c1 & 0xFFu) << (8 * (j & 3));
            w2[j >> 2] |= ((uint32_t)(int)c2 & 0xFFu) << (8 * (j & 3));
          }
          qv[2 * kk] = make_uint4(w1[0], w1[1], w1[2], w1[3]);
          qv[2 * kk + 1] = make_uint4(w2[0], w2[1], w2[2], w2[3]);
        }
      } else {
        // f16 hi + lo of q' * 2^(8 - e), e = exponent of max|q'|: max in
        // [128, 256), about 22 significant bits kept
        const int ex = am > 0.f ? __builtin_amdgcn_frexp_expf(am) : 0;
        if (row_ok) crow = a.qk_scale * ldexpf(1.0f, ex - 8);
#pragma unroll
        for (int kk = 0; kk < T::QSTEPS; ++kk) {
          f16x8 qh16, ql16;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = row_ok ? ldexpf(qrot[r * D + 32 * kk + 8 * g + e], 8 - ex) : 0.f;
            qh16[e] = (_Float16)v;
            ql16[e] = (_Float16)(v - (float)qh16[e]);
          }
          qv[2 * kk] = bitcast<uint4>(qh16);
          qv[2 * kk + 1] = bitcast<uint4>(ql16);
        }
      }
    }
    if constexpr (T::QLDS) {
      __syncthreads();  // every wave has finished reading qrot / the previous segment's store
      if (wave == 0) {
#pragma unroll
        for (int i = 0; i < T::QSTEPS * T::QPIECES; ++i) qst[i * 64 + lane] = qv[i];
      }
      __syncthreads();
    } else {
#pragma unroll
      for (int i = 0; i < T::QSTEPS * T::QPIECES; ++i) qo.reg[i] = qv[i];
      if constexpr (T::QROT) __syncthreads();  // qrot (the merge area) is free again
    }

    // ---- stream this wave's token blocks: blk0 + wave, blk0 + wave + 4, ...
    const uint8_t* head0 = a.pool + (int64_t)h * geo.head_bytes;
    const cint32* bt_row = as_const(a.block_table) + (int64_t)b * a.max_pages;
    float m_run = NEG_INF, l_run = 0.f;
    f32x4 O[T::NT];
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) O[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto qk_phase = [&](const Buf<FMT, D>& buf, int jb, float (&sc)[4]) {
      const int t0 = 16 * jb;
      __builtin_amdgcn_sched_barrier(0);
      const f32x4 S = qk_block<FMT, D>(buf, qo, lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[e] = (t0 + 4 * g + e <= limit) ? S[e] * crow : NEG_INF;
    };
    auto pv_phase = [&](Buf<FMT, D>& buf, int jb, const float (&sc)[4]) {
      const int t0 = 16 * jb;
      const float bm = max_over_g(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
      // The running maximum only has to bound the scores loosely: with it up
      // to RESCALE_SLACK below the true one, p <= 2^RESCALE_SLACK, which f16 P
      // and the fp32 sums hold as well as p <= 1; (m, l, O) stay consistent
      // for whatever m is used.  So l and O are rescaled only on a jump past
      // the slack (and on the first visible block, from m = -inf).
      if (__any(bm > m_run + RESCALE_SLACK)) {
        const float m_new = fmaxf(m_run, bm);
        const float corr = (m_new > m_run) ? fast_exp2(m_run - m_new) : 1.0f;
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
      // a row that has seen no visible key yet has m_run = -inf and only
      // -inf scores: subtract 0 instead so that exp2 gives 0, not NaN
      const float m_use = (m_run == NEG_INF) ? 0.f : m_run;
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = fast_exp2(sc[e] - m_use);
        l_run += p[e];
      }
      const f16x4 P = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
      if (t0 + 16 > L) clear_tail<FMT, D>(buf, L - t0, g);
      // keep the compiler from hoisting every V conversion ahead of the
      // products (it would hold all of them live and spill)
#pragma unroll
      for (int nt = 0; nt < T::NT; ++nt) {
        if ((nt & 3) == 0) __builtin_amdgcn_sched_barrier(0);
        O[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(P, v_operand<FMT, D>(buf, nt, lane), O[nt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    {
      const int jend = blk0 + nblk;
      int j = blk0 + wave;
      if constexpr (T::RING) {
        // this wave's blocks j_k = blk0 + wave + 4 k, k < nk; block k sits in
        // stage k % S, and blocks k + 1 .. k + S - 1 are in flight meanwhile
        constexpr int S = T::RING_S;
        const int nk = nblk > wave ? (nblk - wave + 3) >> 2 : 0;
#pragma unroll
        for (int k = 0; k < S - 1; ++k)
          if (k < nk) stage_block<FMT, D>(ring0 + k * T::STAGE, head0, geo, bt_row, j + 4 * k, lane);
        Buf<FMT, D> A;
        float sc[4];
        int st = 0;
        for (int k = 0; k < nk; ++k) {
          // stage st - 1 (block k - 1) has been read: refill it with block k + S - 1
          if (k + S - 1 < nk) {
            const int sn = st == 0 ? S - 1 : st - 1;
            stage_block<FMT, D>(ring0 + sn * T::STAGE, head0, geo, bt_row, j + 4 * (S - 1), lane);
          }
          wait_staged<T::NDMA, S>(min(S - 1, nk - 1 - k));
          const uint32_t stg = ring0 + st * T::STAGE;
          read_stage_k<FMT, D>(A, stg, lane);
          qk_phase(A, j, sc);
          read_stage_v<FMT, D>(A, stg, lane);
          pv_phase(A, j, sc);
          j += 4;
          st = st + 1 == S ? 0 : st + 1;
        }
      } else if constexpr (T::DOUBLE_BUF) {
        Buf<FMT, D> A, Bb;
        float sc[4];
        if (j < jend) load_block<FMT, D>(A, head0, geo, bt_row, j, lane);
        while (j < jend) {
          if (j + 4 < jend) load_block<FMT, D>(Bb, head0, geo, bt_row, j + 4, lane);
          qk_phase(A, j, sc);
          pv_phase(A, j, sc);
          j += 4;
          if (j >= jend) break;
          if (j + 4 < jend) load_block<FMT, D>(A, head0, geo, bt_row, j + 4, lane);
          qk_phase(Bb, j, sc);
          pv_phase(Bb, j, sc);
          j += 4;
        }
      } else {
        Buf<FMT, D> A;
        float sc[4];
        if (j < jend) load_block<FMT, D>(A, head0, geo, bt_row, j, lane);
        while (j < jend) {
          const int jn = j + 4;
          qk_phase(A, j, sc);
          if (jn < jend) load_k<FMT, D>(A, head0, geo, bt_row, jn, lane);
          pv_phase(A, j, sc);
          if (jn < jend) load_v<FMT, D>(A, head0, geo, bt_row, jn, lane);
          j = jn;
        }
      }
    }

    // ---- merge the 4 waves
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (lane < 16) {
      sm_m[wave * 16 + lane] = m_run;
      sm_l[wave * 16 + lane] = l_run;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 4 * g + e;
      if (row < Rt) {
        float M = NEG_INF;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sm_m[ww * 16 + row]);
        const float mw = sm_m[wave * 16 + row];
        const float f = (mw == NEG_INF) ? 0.f : exp2f(mw - M);
#pragma unroll
        for (int nt = 0; nt < T::NT; ++nt) sm_o[(wave * Rt + row) * D + 16 * nt + c16] = O[nt][e] * f;
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < Rt * D; idx += 256) {
      float o = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) o += sm_o[ww * Rt * D + idx];
      sm_o[idx] = o;  // wave-0 slot of this element; read by this thread only
    }
    __syncthreads();

    // ---- write: one wave per row
    constexpr int E = D / 64;
    const bool direct = whole && a.write_direct;
    for (int row = wave; row < Rt; row += 4) {
      float M = NEG_INF;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sm_m[ww * 16 + row]);
      float l = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float mw = sm_m[ww * 16 + row];
        l += (mw == NEG_INF) ? 0.f : exp2f(mw - M) * sm_l[ww * 16 + row];
      }
      const int rr2 = 16 * rt + row;
      float xo[E];
#pragma unroll
      for (int i = 0; i < E; ++i) xo[i] = sm_o[row * D + E * lane + i];
      if (!direct) {
        const int64_t prow = (int64_t)(u + w) * a.R + rr2;
        float* op = a.ws_o + prow * D + E * lane;
#pragma unroll
        for (int i = 0; i < E; ++i) op[i] = xo[i];
        if (lane == 0) {
          a.ws_ml[prow * 2] = M;
          a.ws_ml[prow * 2 + 1] = l;
        }
      } else {
        const float inv = l > 0.f ? a.v_out_scale / l : 0.f;
#pragma unroll
        for (int i = 0; i < E; ++i) xo[i] *= inv;
        if constexpr (T::VROT) {
          fwht_wave<E>(xo, lane);
#pragma unroll
          for (int i = 0; i < E; ++i) xo[i] *= 0.0625f;
        }
        const int i2 = rr2 / a.G, h2 = h * a.G + (rr2 - i2 * a.G);
        const int64_t orow = ((int64_t)b * a.n_q + i2) * a.H_q + h2;
        float* op = a.out + orow * D + E * lane;
#pragma unroll
        for (int i = 0; i < E; ++i) op[i] = xo[i];
        if (a.lse != nullptr && lane == 0)
          a.lse[orow] = l > 0.f ? (M + __log2f(l)) * 0.69314718055994531f : NEG_INF;
      }
    }
    x = seg_end;
    __syncthreads();  // the next segment reuses the LDS areas
  }
}

// ----------------------------------------------------------- combine
// One workgroup of NT = SG D / 4 threads per (unit, row); thread (g, c) owns
// elements 4c .. 4c + 3 and merges partials g, g + SG, ...
// with a running maximum, rescaling what it holds when the maximum grows
// (the same log-sum-exp merge as the split kernel's); the groups then merge
// through LDS.  Units finished by the split kernel (one workgroup,
// write_direct) are skipped; empty sequences get out = 0, lse = -inf.

template <int D, bool VROT, int SG>
__global__ __launch_bounds__(SG * D / 4) void decode_combine_kernel(DecodeArgs a, int H_kv) {
  constexpr float NEG_INF = -__builtin_inff();
  constexpr int DL = D / 4;       // threads per partial row (4 elements each)
  __shared__ float4 sacc[SG][DL];
  __shared__ float sm[SG], sl[SG];
  const int tid = threadIdx.x, c = tid % DL, g = tid / DL;
  const int u = (int)(blockIdx.x / (unsigned)a.R), rr = (int)(blockIdx.x - (unsigned)u * a.R);
  const int b = u / H_kv, h = u - b * H_kv;
  const int qi = rr / a.G, qh = h * a.G + (rr - qi * a.G);
  const int64_t orow = ((int64_t)b * a.n_q + qi) * a.H_q + qh;
  const int L = a.seq_lens[b];
  const int nb = (L + 15) >> 4;
  if (nb == 0) {
    if (tid < DL) *reinterpret_cast<float4*>(a.out + orow * D + 4 * c) = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.lse != nullptr && tid == 0) a.lse[orow] = NEG_INF;
    return;
  }
  const int total = a.ws_cum[a.B];
  const int per = blocks_per_workgroup(total, a.nwg);
  const int start = a.ws_cum[b] + h * nb;
  const int wa = start / per, wb = (start + nb - 1) / per;
  if (wa == wb && a.write_direct) return;
  const float* ml = a.ws_ml + ((int64_t)(u + wa) * a.R + rr) * 2;
  const float* po = a.ws_o + ((int64_t)(u + wa) * a.R + rr) * D + 4 * c;
  const int nseg = wb - wa + 1;
  const int64_t sml = (int64_t)a.R * 2, so = (int64_t)a.R * D;  // slot strides

  float m = NEG_INF, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto take = [&](float ms, float ls, float4 o) {
    if (ms == NEG_INF) return;  // a partial that saw no visible key
    if (ms > m) {
      const float f = m == NEG_INF ? 0.f : exp2f(m - ms);
      l *= f;
      acc.x *= f; acc.y *= f; acc.z *= f; acc.w *= f;
      m = ms;
    }
    const float w = exp2f(ms - m);
    l += w * ls;
    acc.x += w * o.x; acc.y += w * o.y; acc.z += w * o.z; acc.w += w * o.w;
  };
  int s = g;
  for (; s + SG < nseg; s += 2 * SG) {  // two partials in flight per thread
    const float m0 = ml[s * sml], l0 = ml[s * sml + 1];
    const float m1 = ml[(s + SG) * sml], l1 = ml[(s + SG) * sml + 1];
    const float4 o0 = *reinterpret_cast<const float4*>(po + s * so);
    const float4 o1 = *reinterpret_cast<const float4*>(po + (s + SG) * so);
    take(m0, l0, o0);
    take(m1, l1, o1);
  }
  if (s < nseg) take(ml[s * sml], ml[s * sml + 1], *reinterpret_cast<const float4*>(po + s * so));

  sacc[g][c] = acc;
  if (c == 0) { sm[g] = m; sl[g] = l; }
  __syncthreads();
  if (g != 0) return;
  float M = NEG_INF;
#pragma unroll
  for (int k = 0; k < SG; ++k) M = fmaxf(M, sm[k]);
  float Lt = 0.f;
  float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < SG; ++k) {
    const float w = sm[k] == NEG_INF ? 0.f : exp2f(sm[k] - M);
    const float4 v = sacc[k][c];
    Lt += w * sl[k];
    A.x += w * v.x; A.y += w * v.y; A.z += w * v.z; A.w += w * v.w;
  }
  const float inv = Lt > 0.f ? a.v_out_scale / Lt : 0.f;
  float xv[4] = {A.x * inv, A.y * inv, A.z * inv, A.w * inv};
  if constexpr (VROT) {
    static_assert(D == 256, "the rotation is 256-point");
    fwht_wave<4>(xv, c);  // the 64 threads of group 0 are one wave holding the row
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] *= 0.0625f;
  }
  *reinterpret_cast<float4*>(a.out + orow * D + 4 * c) = make_float4(xv[0], xv[1], xv[2], xv[3]);
  if (a.lse != nullptr && tid == 0) a.lse[orow] = Lt > 0.f ? (M + __log2f(Lt)) * 0.69314718055994531f : NEG_INF;
}

// ----------------------------------------------------------- launchers

#define KVQ_FOR_EACH_DECODE(X)                                                                     \
  X(F_BF16, 128) X(F_BF16, 256) X(F_FP8_ROW, 128) X(F_FP8_ROW, 256) X(F_FP8_TENSOR, 128)          \
  X(F_FP8_TENSOR, 256) X(F_MXFP8, 128) X(F_MXFP8, 256) X(F_INT8_G64, 256) X(F_NVFP4_G16, 256)   \
  X(F_K8V4, 256)

size_t decode_split_lds_bytes(const Geometry& geo, int B, int R) {
#define KVQ_LDS_CASE(F, DD) \
  if (geo.fmt == F && geo.D == DD) return split_lds_bytes<F, DD>(B, R);
  KVQ_FOR_EACH_DECODE(KVQ_LDS_CASE)
#undef KVQ_LDS_CASE
  return 0;
}

hipError_t decode_split_occupancy(const Geometry& geo, int B, int R, int* blocks_per_cu) {
  const size_t lds = decode_split_lds_bytes(geo, B, R);
#define KVQ_OCC_CASE(F, DD)                                                                        \
  if (geo.fmt == F && geo.D == DD)                                                                 \
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, decode_split_kernel<F, DD, false>, \
                                                        256, lds);
  KVQ_FOR_EACH_DECODE(KVQ_OCC_CASE)
#undef KVQ_OCC_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode_split(const Geometry& geo, const DecodeArgs& a, hipStream_t stream) {
  const int tiles = (a.R + 15) / 16;
  const size_t lds = decode_split_lds_bytes(geo, a.B, a.R);
#define KVQ_SPLIT_CASE(F, DD)                                                                                 \
  if (geo.fmt == F && geo.D == DD) {                                                                          \
    if (a.pool_w != nullptr)                                                                                  \
      hipLaunchKernelGGL((decode_split_kernel<F, DD, true>), dim3(a.nwg, tiles), dim3(256), lds, stream, geo, a); \
    else                                                                                                      \
      hipLaunchKernelGGL((decode_split_kernel<F, DD, false>), dim3(a.nwg, tiles), dim3(256), lds, stream, geo, a); \
    return hipGetLastError();                                                                                 \
  }
  KVQ_FOR_EACH_DECODE(KVQ_SPLIT_CASE)
#undef KVQ_SPLIT_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const Geometry& geo, const DecodeArgs& a, hipStream_t stream) {
  const int64_t units = (int64_t)a.B * geo.H_kv;
  const int64_t rows = units * a.R;
  if (rows == 0) return hipSuccess;
  const bool vrot = v_rotated(geo.fmt);
  // partials merged side by side: about the partials per unit, 1 .. 16
  const int64_t expect = a.nwg / units + 1;
  const int sg = expect >= 16 ? 16 : expect >= 8 ? 8 : expect >= 4 ? 4 : expect >= 2 ? 2 : 1;
#define KVQ_COMBINE(DD, VR)                                                                               \
  switch (sg) {                                                                                           \
    case 16: hipLaunchKernelGGL((decode_combine_kernel<DD, VR, 16>), dim3((unsigned)rows), dim3(4 * DD), 0, stream, a, geo.H_kv); break; \
    case 8: hipLaunchKernelGGL((decode_combine_kernel<DD, VR, 8>), dim3((unsigned)rows), dim3(2 * DD), 0, stream, a, geo.H_kv); break; \
    case 4: hipLaunchKernelGGL((decode_combine_kernel<DD, VR, 4>), dim3((unsigned)rows), dim3(DD), 0, stream, a, geo.H_kv); break; \
    case 2: hipLaunchKernelGGL((decode_combine_kernel<DD, VR, 2>), dim3((unsigned)rows), dim3(DD / 2), 0, stream, a, geo.H_kv); break; \
    default: hipLaunchKernelGGL((decode_combine_kernel<DD, VR, 1>), dim3((unsigned)rows), dim3(DD / 4), 0, stream, a, geo.H_kv); break; \
  }
  if (geo.D == 256 && vrot) KVQ_COMBINE(256, true)
  else if (geo.D == 256) KVQ_COMBINE(256, false)
  else if (geo.D == 128 && !vrot) KVQ_COMBINE(128, false)
  else return hipErrorInvalidValue;
#undef KVQ_COMBINE
  return hipGetLastError();
}

}  // namespace kvq
