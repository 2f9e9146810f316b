// kvq_decode_core.hpp -- the per-block pieces of the attention kernels over
// the compressed cache (decode split and chunked prefill): format traits,
// block loads and the LDS ring, the matrix-core operand expanders, Q.K,
// the V operands, the 64-lane FWHT and the softmax helpers.
#pragma once
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kvq_device.hpp"
#include "kvq_internal.hpp"

namespace kvq {

// Every (format, head_dim) the attention kernels are built for.
#define KVQ_FOR_EACH_DECODE(X)                                                                     \
  X(F_BF16, 128) X(F_BF16, 256) X(F_FP8_ROW, 128) X(F_FP8_ROW, 256) X(F_FP8_TENSOR, 128)          \
  X(F_FP8_TENSOR, 256) X(F_MXFP8, 128) X(F_MXFP8, 256) X(F_INT8_G64, 256) X(F_NVFP4_G16, 256)   \
  X(F_K8V4, 256) X(F_MXFP4, 256)

// The (format, head_dim) pairs whose query goes to the matrix cores in two
// pieces, which have a packed kernel for at most 8 rows (VARIANT_PACK).
#define KVQ_FOR_EACH_PACKED(X) X(F_INT8_G64, 256) X(F_NVFP4_G16, 256) X(F_MXFP4, 256)
constexpr int PACK_MAX_ROWS = 8;

template <int FMT, int D>
struct DT {
  static constexpr int KC = k_codec(FMT), VC = v_codec(FMT);
  static constexpr int KBITS = codec_bits(KC), VBITS = codec_bits(VC);
  static constexpr bool QI8 = KC == C_I8G64;    // Q.K on the int8 matrix cores, q in two int8 pieces
  static constexpr bool QF16 = KC == C_E2G16 || KC == C_E2MX;  // Q.K in f16, q split into f16 hi + lo
  static constexpr bool QROT = k_rotated(FMT);  // q is rotated first (K was)
  static constexpr bool VROT = v_rotated(FMT);
  // Q.K on the block-scaled fp8 MFMA, q rounded to MXFP8 (MXFP8 cache only)
  static constexpr bool QMX = (FMT & VARIANT_QMX) != 0;
  static_assert(!QMX || KC == C_E4MX, "the query-MXFP8 variant reads an MXFP8 cache");
  // At most 8 query rows: the query's two pieces share one operand, piece 1
  // in columns 0-7 and piece 2 in columns 8-15 (one lane holds one of them)
  static constexpr bool PACK = (FMT & VARIANT_PACK) != 0;
  static_assert(!PACK || QI8 || QF16, "only a query in two pieces is packed");
  static constexpr int KSTEPS = D / 32;
  static constexpr int QSTEPS = QMX ? D / 128 : QI8 ? D / 64 : D / 32;  // MFMA k-steps of Q.K
  // 16-byte query pieces per k-step and lane (QMX: 32 fp8 codes = two pieces)
  static constexpr int QPIECES = PACK ? 1 : (QI8 || QF16 || QMX) ? 2 : 1;
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
  // RING_LDS bytes per workgroup (two workgroups per CU).  (INT8-G64 first
  // measured faster on its register pipeline; with the start-up and pacing
  // of the current kernel the ring is 4% faster for it too.)
  static constexpr int RING_LDS = 72 * 1024;
  static constexpr int RING_FIT = RING_LDS / (4 * STAGE);
  static constexpr int RING_S = RING_FIT > 4 ? 4 : RING_FIT;
  static constexpr bool RING = RING_S >= 2;
  static_assert(!QMX || RING, "the query-MXFP8 variant reads K from the LDS ring");
  // Without the ring: Q operands in LDS (one ds_read_b128 per k-step) where
  // registers would otherwise spill.
  static constexpr bool QLDS = !RING;
  // Without the ring: prefetch whole blocks into a second register buffer
  // where it fits next to the O accumulators; otherwise reuse one buffer,
  // loading the next block's K as soon as Q.K is done and its V as soon as
  // P.V is done.
  static constexpr bool DOUBLE_BUF = D == 128 || FMT == F_FP8_ROW || FMT == F_FP8_TENSOR;
  static constexpr int NT = D / 16;
  // P.V over pairs of ring blocks with 16x16x32 products (half the products
  // of one block at a time); the first block's V operands wait in registers.
  // For 4-bit V, whose loops are bound by instruction issue (measured: 0-3%
  // faster there, no change for the 8-bit formats); not where the query takes
  // two operand pieces of its own (unpacked), which would spill.
  static constexpr bool PV_PAIR = RING && VBITS == 4 && (QPIECES == 1 || QMX);
  static constexpr int KCH = D * KBITS / 512;                       // 16-B K chunks per lane per block
  static constexpr int VCH = VBITS * NT / 32;                       // 16-B V chunks per lane per block
  // (QMX: one scale byte per 128-value MFMA, one word each)
  static constexpr int KSW = QMX ? D / 128 : KC == C_E4ROW ? 2 : KC == C_I8G64 ? 8 : KC == C_E4MX ? D / 32
                           : KC == C_E2G16 ? 4 : KC == C_E2MX ? D / 128 : 0;
  static constexpr int VSW = VC == C_E4ROW ? 2 : VC == C_I8G64 ? 8 : VC == C_E4MX ? D / 32 : VC == C_E2G16 ? 16
                           : VC == C_E2MX ? D / 32 : 0;
  // K scale bytes of token c16 (4-bit K: the lane's own token, all groups)
  static constexpr int KS_LANE_BYTES = KC == C_E2G16 ? 16 : KC == C_E2MX ? D / 32 : 0;
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

// A 16-byte load with the non-temporal hint (the cache is streamed once per
// launch; see CPOL_STREAM below).
__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

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
  for (int i = 0; i < T::KCH; ++i) buf.k[i] = load_stream16(kc + i * 1024 + lane * 16);
  if constexpr (T::KSW > 0) {
    const uint8_t* ks = ba.hb + geo.off_ks + (int64_t)ba.bip * geo.kscale_blk;
    const int off = T::KS_LANE_BYTES > 0 ? c16 * T::KS_LANE_BYTES : g * (4 * T::KSW);
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
  for (int q = 0; q < T::VCH; ++q) buf.v[q] = load_stream16(vc + q * 1024 + lane * 16);
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

// Cache policy of the copies.  Decode reads every cached byte exactly once
// per launch, so its copies carry the non-temporal hint (NT): on MI355X a
// plain streaming read reaches about 6.0-6.2 TB/s and the same read with NT
// about 6.7-7.0 TB/s, and direct-to-LDS copies gain the same 12% (measured
// with in-bounds read kernels).  Prefill re-reads each block once per row
// tile and relies on the L2 keeping it between them, so it keeps the
// default policy.
constexpr int CPOL_REUSE = 0;
constexpr int CPOL_STREAM = 2;  // the NT bit of the instruction's cache-policy field

template <int BYTES, int CPOL>
__device__ __forceinline__ void copy_plane(uint32_t dst, const uint8_t* src, int lane) {
#pragma unroll
  for (int c = 0; c < BYTES / 1024; ++c)
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(src + c * 1024 + lane * 16),
                                     (lds_void_t*)(uintptr_t)(dst + c * 1024), 16, 0, CPOL);
  constexpr int REM = BYTES % 1024;
  if constexpr (REM > 0) {
    if (lane < REM / 16)  // lane 0 always copies: the instruction is always issued
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(src + (BYTES / 1024) * 1024 + lane * 16),
                                       (lds_void_t*)(uintptr_t)(dst + (BYTES / 1024) * 1024), 16, 0, CPOL);
  }
}

// Start copying the token block at `ba` into the stage at LDS byte address
// `stage`.
template <int FMT, int D, int CPOL = CPOL_STREAM>
__device__ __forceinline__ void stage_block_at(uint32_t stage, const BlockAddr& ba, const Geometry& geo, int lane) {
  using T = DT<FMT, D>;
  copy_plane<T::KB, CPOL>(stage + T::SK, ba.hb + geo.off_kc + (int64_t)ba.bip * T::KB, lane);
  if constexpr (T::KSB > 0)
    copy_plane<T::KSB, CPOL>(stage + T::SKS, ba.hb + geo.off_ks + (int64_t)ba.bip * T::KSB, lane);
  copy_plane<T::VB, CPOL>(stage + T::SV, ba.hb + geo.off_vc + (int64_t)ba.bip * T::VB, lane);
  if constexpr (T::VSB > 0)
    copy_plane<T::VSB, CPOL>(stage + T::SVS, ba.hb + geo.off_vs + (int64_t)ba.bip * T::VSB, lane);
}

// Start copying token block j into the stage at LDS byte address `stage`.
template <int FMT, int D, int CPOL = CPOL_STREAM>
__device__ __forceinline__ void stage_block(uint32_t stage, const uint8_t* head0, const Geometry& geo,
                                            const cint32* bt_row, int j, int lane) {
  stage_block_at<FMT, D, CPOL>(stage, block_addr(head0, geo, bt_row, j), geo, lane);
}

// LDS accesses written in asm that waits for its own LDS counter.  While
// global-to-LDS copies are in flight, the compiler puts a full vmcnt(0) in
// front of every LDS access it emits (it cannot tell the copies' targets
// apart), which would wait for all of them; these leave them in flight.
__device__ __forceinline__ void lds_put4(uint32_t addr, float x0, float x1, float x2, float x3) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = {__float_as_uint(x0), __float_as_uint(x1), __float_as_uint(x2), __float_as_uint(x3)};
  asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_put1(uint32_t addr, float x) {
  asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(addr), "v"(__float_as_uint(x)) : "memory");
}
// x[k][0..7] = the 8 floats at addr + 128 k (k < 8): 16 reads, one wait.
__device__ __forceinline__ void lds_get_8x8(uint32_t addr, float (&x)[8][8]) {
  uint4 r[16];
  asm volatile("ds_read_b128 %0, %16\n\tds_read_b128 %1, %16 offset:16\n\t"
               "ds_read_b128 %2, %16 offset:128\n\tds_read_b128 %3, %16 offset:144\n\t"
               "ds_read_b128 %4, %16 offset:256\n\tds_read_b128 %5, %16 offset:272\n\t"
               "ds_read_b128 %6, %16 offset:384\n\tds_read_b128 %7, %16 offset:400\n\t"
               "ds_read_b128 %8, %16 offset:512\n\tds_read_b128 %9, %16 offset:528\n\t"
               "ds_read_b128 %10, %16 offset:640\n\tds_read_b128 %11, %16 offset:656\n\t"
               "ds_read_b128 %12, %16 offset:768\n\tds_read_b128 %13, %16 offset:784\n\t"
               "ds_read_b128 %14, %16 offset:896\n\tds_read_b128 %15, %16 offset:912\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
                 "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]),
                 "=&v"(r[14]), "=&v"(r[15])
               : "v"(addr) : "memory");
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint4 lo = r[2 * k], hi = r[2 * k + 1];
    x[k][0] = __uint_as_float(lo.x); x[k][1] = __uint_as_float(lo.y); x[k][2] = __uint_as_float(lo.z);
    x[k][3] = __uint_as_float(lo.w); x[k][4] = __uint_as_float(hi.x); x[k][5] = __uint_as_float(hi.y);
    x[k][6] = __uint_as_float(hi.z); x[k][7] = __uint_as_float(hi.w);
  }
}

// Four 8-byte reads at addr + 512 i (i < 4), waiting for them.
__device__ __forceinline__ void lds_get_rows4(uint32_t addr, uint2 (&x)[4]) {
  asm volatile("ds_read_b64 %0, %4\n\tds_read_b64 %1, %4 offset:512\n\tds_read_b64 %2, %4 offset:1024\n\t"
               "ds_read_b64 %3, %4 offset:1536\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]) : "v"(addr) : "memory");
}
__device__ __forceinline__ float lds_get1(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(addr) : "memory");
  return __uint_as_float(v);
}

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt fields at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until every copy of a block is done when `after` blocks (wave-
// uniform, < S) were staged behind it.  Copies complete in order, so
// vmcnt(after * NDMA) suffices; a count past the counter's 6 bits waits at
// 63, which is only more than needed.
template <int NDMA, int S, int A = S - 1>
__device__ __forceinline__ void wait_staged(int after) {
  if constexpr (A > 0) {
    if (after >= A) {
      wait_vmcnt<(A * NDMA < 63 ? A * NDMA : 63)>();
      return;
    }
    wait_staged<NDMA, S, A - 1>(after);
  } else {
    wait_vmcnt<0>();
  }
}

// NC 16-byte code chunks at c + i * CS (i < NC) and SW scale words at s
// (consecutive), read from LDS in one asm block that waits for them.
template <int NC, int CS, int SW>
__device__ __forceinline__ void lds_read_part(uint4 (&c)[NC], uint32_t (&w)[SW > 0 ? SW : 1], uint32_t ca,
                                              uint32_t sa) {
  if constexpr (NC == 8) {  // 16-bit codes at D = 256 (no scales): two reads of 4
    static_assert(SW == 0, "");
    uint4 (&lo)[4] = *reinterpret_cast<uint4 (*)[4]>(&c[0]);
    uint4 (&hi)[4] = *reinterpret_cast<uint4 (*)[4]>(&c[4]);
    lds_read_part<4, CS, 0>(lo, w, ca, sa);
    lds_read_part<4, CS, 0>(hi, w, ca + 4 * CS, sa);
    return;
  }
  static_assert(NC == 2 || NC == 4 || NC == 8, "");
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

// Operands of the block-scaled 16x16x128 fp8 MFMA, for NS MFMAs (128
// head_dim values each).  The instruction's lane layout (measured): lane
// 16 i + x holds row x (A: token, B: query row) at MFMA k = 16 i + j in bytes
// j < 16 and k = 64 + 16 i + (j - 16) in bytes j >= 16, and gives the scale of
// k-block m = i (k in [32 i, 32 i + 32)) for row x.  MFMA s takes
// d = 128 s + k, so k-block m is the MX group 4 s + m.  From the K tile order
// (8 values of k-step kk for token t per 8-byte run, at byte
// (kk / 2) * 1024 + (g' * 16 + t) * 16 + (kk % 2) * 8), the lane's four 8-byte
// runs of MFMA s are at (2 s + hh) * 1024 + ((2 (i % 2) + u) * 16 + t) * 16
// + (i / 2) * 8 (bytes 8 (2 hh + u) ..), and its scale is the byte of token t,
// group 4 s + i.  One asm block that waits for its own reads (see
// lds_read_part).
template <int NS>
__device__ __forceinline__ void lds_read_qmx(uint4 (&c)[2 * NS], uint32_t (&w)[NS], uint32_t ca, uint32_t sa) {
  static_assert(NS == 1 || NS == 2, "head_dim 128 or 256");
  uint2 r[4 * NS];
  if constexpr (NS == 1) {
    asm volatile("ds_read_b64 %0, %5\n\tds_read_b64 %1, %5 offset:256\n\t"
                 "ds_read_b64 %2, %5 offset:1024\n\tds_read_b64 %3, %5 offset:1280\n\t"
                 "ds_read_u8 %4, %6\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(w[0])
                 : "v"(ca), "v"(sa) : "memory");
  } else {
    asm volatile("ds_read_b64 %0, %10\n\tds_read_b64 %1, %10 offset:256\n\t"
                 "ds_read_b64 %2, %10 offset:1024\n\tds_read_b64 %3, %10 offset:1280\n\t"
                 "ds_read_b64 %4, %10 offset:2048\n\tds_read_b64 %5, %10 offset:2304\n\t"
                 "ds_read_b64 %6, %10 offset:3072\n\tds_read_b64 %7, %10 offset:3328\n\t"
                 "ds_read_u8 %8, %11\n\tds_read_u8 %9, %11 offset:4\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
                   "=&v"(r[7]), "=&v"(w[0]), "=&v"(w[1])
                 : "v"(ca), "v"(sa) : "memory");
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    c[2 * s] = make_uint4(r[4 * s].x, r[4 * s].y, r[4 * s + 1].x, r[4 * s + 1].y);
    c[2 * s + 1] = make_uint4(r[4 * s + 2].x, r[4 * s + 2].y, r[4 * s + 3].x, r[4 * s + 3].y);
  }
}

// The K codes and scales of the block in `stage`, in the registers and lane
// order load_k would give (QMX: in the block-scaled MFMA's order).
template <int FMT, int D>
__device__ __forceinline__ void read_stage_k(Buf<FMT, D>& buf, uint32_t stage, int lane) {
  using T = DT<FMT, D>;
  const int g = lane >> 4, c16 = lane & 15;
  if constexpr (T::QMX) {
    lds_read_qmx<D / 128>(buf.k, buf.ks, stage + T::SK + ((2 * (g & 1)) * 16 + c16) * 16 + (g >> 1) * 8,
                          stage + T::SKS + c16 * (D / 32) + g);
  } else {
    const uint32_t sa = stage + T::SKS + (T::KS_LANE_BYTES > 0 ? c16 * T::KS_LANE_BYTES : g * (4 * T::KSW));
    lds_read_part<T::KCH, 1024, T::KSW>(buf.k, buf.ks, stage + T::SK + lane * 16, sa);
  }
}

// The V codes and scales of the block in `stage`, as load_v would give them.
template <int FMT, int D>
__device__ __forceinline__ void read_stage_v(Buf<FMT, D>& buf, uint32_t stage, int lane) {
  using T = DT<FMT, D>;
  const int g = lane >> 4;
  lds_read_part<T::VCH, 1024, T::VSW>(buf.v, buf.vs, stage + T::SV + lane * 16, stage + T::SVS + g * (4 * T::VSW));
}

// One 16-byte LDS write that waits for itself (see lds_read_part).
__device__ __forceinline__ void lds_put16(uint32_t addr, uint4 v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = {v.x, v.y, v.z, v.w};
  asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(addr), "v"(w) : "memory");
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

// 8 E2M1 codes times 2^(byte - 127) (UE8M0): the scaled conversion adds the
// scale's exponent, so the f16 result is exact while code x scale stays in
// f16 range.  Byte 0 is taken as 2^-126 (the conversion needs a normal fp32
// scale); such a group holds values far below f16's range either way.
__device__ __forceinline__ f16x8 e2m1x8_f16_mx(uint32_t w, uint32_t byte) {
  const float sc = __uint_as_float((byte > 1u ? byte : 1u) << 23);
  uint4 r;
  r.x = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 0));
  r.y = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 1));
  r.z = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 2));
  r.w = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 3));
  return bitcast<f16x8>(r);
}

__device__ __forceinline__ uint32_t word(const uint4& q, int i) {
  return i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w;
}

// ----------------------------------------------------------- Q operands

template <int FMT, int D, bool IN_LDS = DT<FMT, D>::QLDS>
struct QOps {
  // B operands of S = K . Q^T, k-step kk, piece p (bf16 q; f16 hi, lo; or
  // int8 coarse, fine), as raw 16-byte lane values, in registers or in LDS
  using T = DT<FMT, D>;
  uint4 reg[IN_LDS ? 1 : T::QSTEPS * T::QPIECES];
  uint32_t qsc[T::QMX ? T::QSTEPS : 1];  // QMX: q's UE8M0 this lane gives MFMA s (in bits 0..7)
  const uint4* lds;
  int lane;
  __device__ __forceinline__ uint4 get(int kk, int p) const {
    if constexpr (IN_LDS) return lds[(kk * T::QPIECES + p) * 64 + lane];
    else return reg[kk * T::QPIECES + p];
  }
};

// ----------------------------------------------------------- S = K . Q^T

template <int FMT, int D, typename Q>
__device__ __forceinline__ f32x4 qk_block(const Buf<FMT, D>& buf, const Q& qo, int lane) {
  using T = DT<FMT, D>;
  f32x4 S = {0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  if constexpr (T::QMX) {
    // E4M3 x E4M3 with both UE8M0 scales applied by the instruction (A and B
    // format 0 = E4M3; scale byte 0 of each lane's word)
#pragma unroll
    for (int s = 0; s < T::QSTEPS; ++s) {
      const uint4 k0 = buf.k[2 * s], k1 = buf.k[2 * s + 1];
      const uint4 q0 = qo.get(s, 0), q1 = qo.get(s, 1);
      const i32x8 a = {(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w, (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
      const i32x8 bq = {(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w};
      S = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bq, S, 0, 0, 0, (int)buf.ks[s], 0, (int)qo.qsc[s]);
    }
  } else if constexpr (T::KC == C_BF16) {
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
    if constexpr (T::PACK) {
      // columns 0-7 hold the coarse digits, 8-15 the fine ones: weigh this
      // lane's sums by 254 or 1, then add the other half's (lane c ^ 8)
      const float w = (lane & 8) ? 1.0f : 254.0f;
#pragma unroll
      for (int grp = 0; grp < T::KCH; ++grp) {
        const i32x4 a = __builtin_amdgcn_mfma_i32_16x16x64_i8(bitcast<i32x4>(buf.k[grp]),
                                                             bitcast<i32x4>(qo.get(grp, 0)), izero, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int hw = e * 4 + grp;  // halfword of token 4g+e, group grp
          const float sc = f16_bits_to_f32((buf.ks[hw >> 1] >> (16 * (hw & 1))) & 0xFFFFu);
          S[e] += (float)a[e] * sc;  // |a| <= 64*127*127: exact in fp32
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S[e] *= w;
        S[e] += quad_swap<ROW_ROR8>(S[e]);
      }
    } else {
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
    }
  } else if constexpr (T::KC == C_E2G16) {
    // E2M1 x UE4M3 is exact in f16: fold the group scale into the operand.
    // lane (g, t): k-step kk covers d in [32kk + 8g, +8) -> group 2kk + g/2
    const int gb = (lane >> 5) & 1;
    f32x4 S1 = zero;
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
        if constexpr (T::PACK) {
          // hi (columns 0-7) and lo (8-15) in one product; two chains by k-step
          if (hh & 1) S1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bitcast<f16x8>(qo.get(kk, 0)), S1, 0, 0, 0);
          else S = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bitcast<f16x8>(qo.get(kk, 0)), S, 0, 0, 0);
        } else {
          // hi and lo parts of q in separate chains
          S = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bitcast<f16x8>(qo.get(kk, 0)), S, 0, 0, 0);
          S1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bitcast<f16x8>(qo.get(kk, 1)), S1, 0, 0, 0);
        }
      }
    }
    S += S1;
    if constexpr (T::PACK) {
#pragma unroll
      for (int e = 0; e < 4; ++e) S[e] += quad_swap<ROW_ROR8>(S[e]);  // hi + lo of row c16 % 8
    }
  } else if constexpr (T::KC == C_E2MX) {
    // one UE8M0 per 32 values = per k-step, of the lane's token (lane % 16),
    // applied by the conversion itself; q' as f16 hi + lo as for NVFP4
    f32x4 S1 = zero;
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) {
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        const int kk = 4 * i + hh;
        const f16x8 a = e2m1x8_f16_mx(word(buf.k[i], hh), (buf.ks[kk >> 2] >> (8 * (kk & 3))) & 0xFFu);
        if constexpr (T::PACK) {
          if (hh & 1) S1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bitcast<f16x8>(qo.get(kk, 0)), S1, 0, 0, 0);
          else S = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bitcast<f16x8>(qo.get(kk, 0)), S, 0, 0, 0);
        } else {
          S = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bitcast<f16x8>(qo.get(kk, 0)), S, 0, 0, 0);
          S1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bitcast<f16x8>(qo.get(kk, 1)), S1, 0, 0, 0);
        }
      }
    }
    S += S1;
    if constexpr (T::PACK) {
#pragma unroll
      for (int e = 0; e < 4; ++e) S[e] += quad_swap<ROW_ROR8>(S[e]);
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
  } else if constexpr (T::VC == C_E2MX) {
    // codes as for NVFP4; the UE8M0 of tokens 4g .. 4g + 3 for group nt / 2
    // (byte e of word nt / 2) as exact f16 powers of two (in f16 range)
    const uint32_t w = word(buf.v[nt >> 3], (nt & 7) >> 1);
    f16x2 a, b;
    if (nt & 1) {
      a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
      b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
    } else {
      a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
      b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    }
    const uint32_t sw = buf.vs[nt >> 1];
    auto pow2 = [](uint32_t byte) { return __uint_as_float(byte << 23); };  // 2^(byte - 127); 0 for byte 0
    const f16x2 s01 = __builtin_amdgcn_cvt_pkrtz(pow2(sw & 0xFFu), pow2((sw >> 8) & 0xFFu));
    const f16x2 s23 = __builtin_amdgcn_cvt_pkrtz(pow2((sw >> 16) & 0xFFu), pow2(sw >> 24));
    a *= s01;
    b *= s23;
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

// Unnormalized Hadamard of a 64*E vector, lane l holding elements
// E*l .. E*l+E-1 (any fp32 order is fine on the read path).  No LDS: the
// cross-lane stages are register permutations, so a transform costs a few
// dozen instructions instead of a chain of LDS round trips.  Needs the
// whole wave active.
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
  for (int i = 0; i < E; ++i) {
    x[i] = xlane_butterfly<1>(x[i], lane);
    x[i] = xlane_butterfly<2>(x[i], lane);
    x[i] = xlane_butterfly<4>(x[i], lane);
    x[i] = xlane_butterfly<8>(x[i], lane);
    x[i] = xlane_butterfly<16>(x[i], lane);
    x[i] = xlane_butterfly<32>(x[i], lane);
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

// Sum over the four lanes 16 g + c (g = 0..3) that share c (same swaps as
// max_over_g; every lane gets the sum).
__device__ __forceinline__ float sum_over_g(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(bitcast<uint32_t>(x), bitcast<uint32_t>(x), false, false);
  x = bitcast<float>((uint32_t)a[0]) + bitcast<float>((uint32_t)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(bitcast<uint32_t>(x), bitcast<uint32_t>(x), false, false);
  return bitcast<float>((uint32_t)b[0]) + bitcast<float>((uint32_t)b[1]);
}

// Maximum over the whole wave (every lane gets it); needs the whole wave active.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, lane_xor<1>(x));
  x = fmaxf(x, lane_xor<2>(x));
  x = fmaxf(x, lane_xor<4>(x));
  x = fmaxf(x, lane_xor<8>(x));
  return max_over_g(x);
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
  } else if constexpr (T::VC == C_E2G16 || T::VC == C_E2MX) {  // byte e of each word: token 4g + e
#pragma unroll
    for (int w = 0; w < T::VSW; ++w) buf.vs[w] &= bmask;
  }
}

}  // namespace kvq
