// kvq_prefill.hip -- chunked-prefill causal attention over the compressed
// paged cache.  After a prefill chunk of n_q tokens has been appended to each
// sequence (the write path), every one of its query tokens attends to all
// cached positions up to its own (NInfer KV-cache guide: the causal attention
// over the cache that prefill chunks run; the quantity is the one decode
// computes, with n_q up to the chunk length).
//
// Decode spreads one unit's blocks over many workgroups; prefill has rows to
// spare instead (G * n_q per kv head, 12288 for a 2048-token chunk at G = 6),
// so nothing is split: a workgroup takes 64 rows of one (sequence b, kv head
// h) unit, 16 per wave, and walks the unit's blocks up to its rows' last
// visible position.  Wave 0 copies each block once into the workgroup's LDS
// ring; one barrier per block publishes it and frees the stage read last;
// every wave then runs the decode kernel's per-block code on it for its own
// rows (K expanded exactly into matrix-core operands, Q.K, online softmax
// with the lazy running maximum, P.V).  Work items (row tiles) go out in
// unit-major order, one workgroup each; the hardware hands workgroups to the
// 8 XCDs round robin, so every XCD gets every eighth tile of every unit and
// the XCDs' shares stay even whatever the length mix, while the tiles of a
// unit that one XCD runs side by side still share its L2.  (Keeping a unit's
// tiles on one XCD left one XCD with 1.66 times the mean work on 64 mixed
// lengths.)  Each wave finishes its own
// rows: normalization, the inverse rotation of V for the rotated formats
// (through LDS, 8 rows at a time), output and lse.
#include <hip/hip_runtime.h>

#include "kvq_decode_core.hpp"

namespace kvq {

// The workgroup's block ring: up to 4 stages within 64 KB (deeper rings
// measured slower).  V codes that need expanding (all but fp16 V) are
// expanded once per block for the four waves: two buffers of f16 B operands
// of the 16x16x16 P.V products, [pair of n-tiles][lane] 16 bytes each, after
// the ring.  With them two workgroups fit a CU.  Outside the block loop the
// same area holds 8 fp32 rows of D per wave.
template <int FMT, int D>
struct PT {
  using T = DT<FMT, D>;
  static constexpr int FIT = 64 * 1024 / T::STAGE;
  static constexpr int S = FIT > 4 ? 4 : FIT;
  static_assert(S >= 2, "the ring keeps a block in flight while one is read");
  static constexpr bool VSH = T::VC != C_F16;
  static_assert(!VSH || S >= 3, "blocks k (K) and k + 1 (V) are read while k + 2 is in flight");
  static constexpr int VBUF = T::NT * 64 * 8;  // one block's f16 V operands
  static constexpr int RING_BYTES = S * T::STAGE + (VSH ? 2 * VBUF : 0);
  static constexpr int ROWS_BYTES = 4 * 8 * D * 4;  // 8 fp32 rows per wave
  static constexpr int AREA = RING_BYTES > ROWS_BYTES ? RING_BYTES : ROWS_BYTES;
  static constexpr int HDR_FLOATS = 256;  // per wave 16 m, 16 l, 16 q maxima (4 waves)
};

template <int FMT, int D>
__host__ __device__ constexpr size_t prefill_lds_bytes() {
  return PT<FMT, D>::HDR_FLOATS * sizeof(float) + (size_t)PT<FMT, D>::AREA;
}

// One work item = 64 rows (a row tile) of one unit, item n on workgroup n.
template <int FMT, int D>
__global__ __launch_bounds__(256, 2) void prefill_kernel(Geometry geo, DecodeArgs a, int tiles) {
  using T = DT<FMT, D>;
  using PP = PT<FMT, D>;
  constexpr float NEG_INF = -__builtin_inff();
  constexpr int E = D / 64;
  extern __shared__ float lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int wi = blockIdx.x;
  const int u = wi / tiles, tile = wi - u * tiles;
  const int b = u / geo.H_kv, h = u - b * geo.H_kv;
  const int L = as_const(a.seq_lens)[b];

  float* hdr = lds + wave * 48;  // m [16], l [16], q maxima [16] of this wave's rows
  uint8_t* area = reinterpret_cast<uint8_t*>(lds + PP::HDR_FLOATS);
  float* wbuf = reinterpret_cast<float*>(area) + wave * 8 * D;  // this wave's 8 rows, outside the block loop
  const uint32_t ring0 = (uint32_t)(uintptr_t)(void*)area;     // the ring during it

  // ---- this wave's rows r0 .. r0 + 15; lane row c16 (S layout) -> (query i, head)
  const int r0 = 64 * tile + 16 * wave;
  const bool has_rows = r0 < a.R;  // wave-uniform; a wave without rows still joins the barriers
  const int rr = r0 + c16;
  const bool row_ok = rr < a.R;
  const int qi = rr / a.G, qh = h * a.G + (rr - qi * a.G);
  const int limit = row_ok ? L - a.n_q + qi : -1;  // last visible position of the row
  // blocks the workgroup walks: up to the last visible position of its last row
  const int last_row = min(a.R, 64 * tile + 64) - 1;
  const int lim_wg = L - a.n_q + last_row / a.G;
  const int nk = lim_wg >= 0 ? (lim_wg >> 4) + 1 : 0;

  // ---- Q operands of the wave's rows (as the decode kernel's, per wave)
  QOps<FMT, D, false> qo;
  qo.lane = lane;
  qo.lds = nullptr;
  float crow = a.qk_scale;
  if constexpr (!T::QROT) {
    const uint16_t* qp = a.q + (((int64_t)b * a.n_q + qi) * a.H_q + qh) * D;
#pragma unroll
    for (int kk = 0; kk < T::QSTEPS; ++kk) {
      uint4 q4 = make_uint4(0, 0, 0, 0);
      if (row_ok) q4 = *reinterpret_cast<const uint4*>(qp + 32 * kk + 8 * g);
      qo.reg[kk] = q4;
    }
  } else {
    // q' = H q / 16 in fp32, 8 rows at a time through wbuf; the lanes whose
    // row is in the pass build their operands from it
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll 1
      for (int r = 0; r < 8; ++r) {
        const int rr2 = r0 + 8 * pass + r;
        float xq[E];
#pragma unroll
        for (int i = 0; i < E; ++i) xq[i] = 0.f;
        if (rr2 < a.R) {  // wave-uniform
          const int i2 = rr2 / a.G, h2 = h * a.G + (rr2 - i2 * a.G);
          const uint2 q2 = *reinterpret_cast<const uint2*>(a.q + (((int64_t)b * a.n_q + i2) * a.H_q + h2) * D + E * lane);
          xq[0] = bf16_to_f32(q2.x & 0xFFFFu); xq[1] = bf16_to_f32(q2.x >> 16);
          xq[2] = bf16_to_f32(q2.y & 0xFFFFu); xq[3] = bf16_to_f32(q2.y >> 16);
          fwht_wave<E>(xq, lane);
        }
        float am = 0.f;
#pragma unroll
        for (int i = 0; i < E; ++i) { xq[i] *= 0.0625f; am = fmaxf(am, fabsf(xq[i])); }
        am = wave_max(am);
#pragma unroll
        for (int i = 0; i < E; ++i) wbuf[r * D + E * lane + i] = xq[i];
        if (lane == 0) hdr[32 + 8 * pass + r] = am;
      }
      if ((c16 >> 3) == pass) {
        const float* qrow = wbuf + (c16 & 7) * D;
        const float am = row_ok ? hdr[32 + c16] : 0.f;
        if constexpr (T::QI8) {
          const float inv = am > 0.f ? 127.0f / am : 0.f;
          crow = am > 0.f ? a.qk_scale * (am / (127.0f * 254.0f)) : 0.f;
#pragma unroll
          for (int kk = 0; kk < T::QSTEPS; ++kk) {
            uint32_t w1[4] = {0, 0, 0, 0}, w2[4] = {0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int d = 64 * kk + (j < 8 ? 8 * g + j : 32 + 8 * g + (j - 8));
              const float v = row_ok ? qrow[d] * inv : 0.f;
              const float c1 = fmaxf(fminf(rintf(v), 127.f), -127.f);
              const float c2 = fmaxf(fminf(rintf((v - c1) * 254.0f), 127.f), -127.f);
              w1[j >> 2] |= ((uint32_t)(int)c1 & 0xFFu) << (8 * (j & 3));
              w2[j >> 2] |= ((uint32_t)(int)c2 & 0xFFu) << (8 * (j & 3));
            }
            qo.reg[2 * kk] = make_uint4(w1[0], w1[1], w1[2], w1[3]);
            qo.reg[2 * kk + 1] = make_uint4(w2[0], w2[1], w2[2], w2[3]);
          }
        } else {
          const int ex = am > 0.f ? __builtin_amdgcn_frexp_expf(am) : 0;
          if (row_ok) crow = a.qk_scale * ldexpf(1.0f, ex - 8);
#pragma unroll
          for (int kk = 0; kk < T::QSTEPS; ++kk) {
            f16x8 qh16, ql16;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float v = row_ok ? ldexpf(qrow[32 * kk + 8 * g + e], 8 - ex) : 0.f;
              qh16[e] = (_Float16)v;
              ql16[e] = (_Float16)(v - (float)qh16[e]);
            }
            qo.reg[2 * kk] = bitcast<uint4>(qh16);
            qo.reg[2 * kk + 1] = bitcast<uint4>(ql16);
          }
        }
      }
    }
  }
  // every wave is done with its rows in the area before the ring's copies overwrite it
  __syncthreads();

  // ---- stream the unit's blocks 0 .. nk - 1 through this wave's ring
  const uint8_t* head0 = a.pool + (int64_t)h * geo.head_bytes;
  const cint32* bt_row = as_const(a.block_table) + (int64_t)b * a.max_pages;
  float m_run = NEG_INF, l_run = 0.f;
  f32x4 O[T::NT];
#pragma unroll
  for (int nt = 0; nt < T::NT; ++nt) O[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    // Wave 0 copies blocks 0 .. S - 2 ahead, block k into stage k % S.
    // Without shared V: in iteration k it waits for block k, the barrier
    // publishes it (and every wave is then done with block k - 1), and wave
    // 0 refills that stage with block k + S - 1.  With shared V, block k + 1
    // is what wave 0 waits for: after the barrier every wave expands a
    // quarter of block k + 1's V operands into buffer (k + 1) & 1, while the
    // products of block k read K from its stage and V from buffer k & 1
    // (filled the iteration before, published by this barrier).
    constexpr int S = PP::S;
    const uint32_t vexp0 = ring0 + S * T::STAGE;
    auto expand_v = [&](int kb) {
      Buf<FMT, D> Vb;
      read_stage_v<FMT, D>(Vb, ring0 + (kb % S) * T::STAGE, lane);
      if (16 * kb + 16 > L) clear_tail<FMT, D>(Vb, L - 16 * kb, g);
      const uint32_t dst = vexp0 + (kb & 1) * PP::VBUF;
      constexpr int PER = T::NT / 4;  // n-tiles per wave (a constant index keeps Vb in registers)
#pragma unroll
      for (int nt = 0; nt < T::NT; nt += 2) {
        if (nt / PER != wave) continue;  // wave-uniform
        const f16x4 va = v_operand<FMT, D>(Vb, nt, lane), vb = v_operand<FMT, D>(Vb, nt + 1, lane);
        lds_put16(dst + (uint32_t)(((nt >> 1) * 64 + lane) * 16),
                  make_uint4(bitcast<uint2>(va).x, bitcast<uint2>(va).y, bitcast<uint2>(vb).x, bitcast<uint2>(vb).y));
      }
    };
    if (wave == 0) {
#pragma unroll
      for (int k = 0; k < S - 1; ++k)
        if (k < nk) stage_block<FMT, D, CPOL_REUSE>(ring0 + k * T::STAGE, head0, geo, bt_row, k, lane);
    }
    if constexpr (PP::VSH) {
      if (nk > 0) {
        if (wave == 0) wait_staged<T::NDMA, S>(min(S - 2, nk - 1));
        __syncthreads();
        expand_v(0);
      }
    }
    Buf<FMT, D> A;
    int st = 0;
    for (int k = 0; k < nk; ++k) {
      if constexpr (PP::VSH) {
        if (wave == 0 && k + 1 < nk) wait_staged<T::NDMA, S>(min(S - 3, nk - 2 - k));
      } else {
        if (wave == 0) wait_staged<T::NDMA, S>(min(S - 2, nk - 1 - k));
      }
      __syncthreads();
      if (wave == 0 && k + S - 1 < nk)
        stage_block<FMT, D, CPOL_REUSE>(ring0 + ((st + S - 1) % S) * T::STAGE, head0, geo, bt_row, k + S - 1, lane);
      const uint32_t stg = ring0 + st * T::STAGE;
      st = st + 1 == S ? 0 : st + 1;
      if constexpr (PP::VSH) {
        if (k + 1 < nk) expand_v(k + 1);
      }
      if (!has_rows) continue;
      const int t0 = 16 * k;
      read_stage_k<FMT, D>(A, stg, lane);
      __builtin_amdgcn_sched_barrier(0);
      const f32x4 Sx = qk_block<FMT, D>(A, qo, lane);
      __builtin_amdgcn_sched_barrier(0);
      float sc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[e] = (t0 + 4 * g + e <= limit) ? Sx[e] * crow : NEG_INF;
      if constexpr (!PP::VSH) read_stage_v<FMT, D>(A, stg, lane);
      // online softmax with the lazy running maximum (decode kernel's rule)
      const float bm = max_over_g(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
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
      const float m_use = (m_run == NEG_INF) ? 0.f : m_run;
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = fast_exp2(sc[e] - m_use);
        l_run += p[e];
      }
      const f16x4 P = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
      if constexpr (PP::VSH) {
        const uint32_t src = vexp0 + (k & 1) * PP::VBUF + lane * 16;
#pragma unroll
        for (int h = 0; h < T::NT / 8; ++h) {  // 8 n-tiles (4 pairs) per read
          uint4 v4[4];
          uint32_t none[1];
          lds_read_part<4, 1024, 0>(v4, none, src + h * 4096, 0);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint2 w = (i & 1) ? make_uint2(v4[i >> 1].z, v4[i >> 1].w) : make_uint2(v4[i >> 1].x, v4[i >> 1].y);
            O[8 * h + i] = __builtin_amdgcn_mfma_f32_16x16x16f16(P, bitcast<f16x4>(w), O[8 * h + i], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        if (t0 + 16 > L) clear_tail<FMT, D>(A, L - t0, g);
#pragma unroll
        for (int nt = 0; nt < T::NT; ++nt) {
          if ((nt & 3) == 0) __builtin_amdgcn_sched_barrier(0);
          O[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(P, v_operand<FMT, D>(A, nt, lane), O[nt], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();  // every wave is done with the ring before the area holds rows again
  if (!has_rows) return;

  // ---- finish the rows: l over the row's 4 lane groups; row 4g + e of O
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (lane < 16) {
    hdr[lane] = m_run;
    hdr[16 + lane] = l_run;
  }
  float inv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float l = hdr[16 + 4 * g + e];
    inv[e] = l > 0.f ? a.v_out_scale / l : 0.f;
  }
  auto out_row = [&](int r) -> int64_t {  // output row of wave row r
    const int rr2 = r0 + r;
    const int i2 = rr2 / a.G, h2 = h * a.G + (rr2 - i2 * a.G);
    return ((int64_t)b * a.n_q + i2) * a.H_q + h2;
  };
  if constexpr (T::VROT) {
    // o = H o' / 16 per row, 8 rows at a time through wbuf (the idle ring)
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 4 * g + e;
        if ((row >> 3) == pass) {
#pragma unroll
          for (int nt = 0; nt < T::NT; ++nt) wbuf[(row & 7) * D + 16 * nt + c16] = O[nt][e] * inv[e];
        }
      }
#pragma unroll 1
      for (int r = 0; r < 8; ++r) {
        const int row = 8 * pass + r;
        float xo[E];
#pragma unroll
        for (int i = 0; i < E; ++i) xo[i] = wbuf[r * D + E * lane + i];
        fwht_wave<E>(xo, lane);
        if (r0 + row < a.R) {
          float* op = a.out + out_row(row) * D + E * lane;
#pragma unroll
          for (int i = 0; i < E; ++i) op[i] = xo[i] * 0.0625f;
        }
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 4 * g + e;
      if (r0 + row < a.R) {
        float* op = a.out + out_row(row) * D + c16;
#pragma unroll
        for (int nt = 0; nt < T::NT; ++nt) op[16 * nt] = O[nt][e] * inv[e];
      }
    }
  }
  if (a.lse != nullptr && lane < 16 && row_ok)
    a.lse[out_row(lane)] = l_run > 0.f ? (m_run + __log2f(l_run)) * 0.69314718055994531f : NEG_INF;
}

// ---------------------------------------------------------------- 32-row waves
//
// For the formats whose K expands exactly to bf16 with the raw query as the
// other operand (BF16; FP8-row and K8V4 with the row scale applied to the
// scores; FP8-tensor with its scale folded into the score scale; MXFP8 with
// its power-of-two group scale folded into the conversion), a wave takes 32
// query rows and the products are the 32x32x16 matrix instructions, which
// the 16-row shapes reach only half of the rate of.  Both products are taken
// transposed, S^T = K Q^T and O^T = V^T P^T, so that the query row is the
// MFMA column: lane l owns row l % 32 (lanes l and l + 32 share it), and the
// running maximum, the sum and the rescale of O stay in the lane.
//
// Operand orders.  In an A (B) operand lane l holds row (column) l % 32 and
// the 8 k-values of half l / 32.  S^T's rows are tokens: the K operand's
// row rho holds token tau(rho), rho with bits 2 and 3 swapped, so that
// register 8 m + i of S^T holds token 16 m + 8 (l / 32) + i, which is then
// already the P^T operand of the P.V product over tokens 16 m .. 16 m + 15.
// The V^T operand (dims x tokens) comes from a buffer the workgroup fills
// once per 32-token step: [block m][half h][dim d][tokens 8 h .. 8 h + 7]
// f16, so that the 32 lanes of a half read 512 consecutive bytes.
//
// Pipeline: a ring of S stages of two 16-token blocks, each step's copies
// spread over the four waves; one barrier per step publishes a stage.  All
// 256 threads expand V codes into the buffer: with two buffers (where a
// 3-stage ring fits beside them) the next step's, during this one; with one
// buffer this step's, published by a second barrier before P.V.

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

template <int FMT>
constexpr bool wide_prefill_format() {
  return k_codec(FMT) == C_BF16 || k_codec(FMT) == C_E4ROW || k_codec(FMT) == C_E4TEN || k_codec(FMT) == C_E4MX;
}

template <int FMT, int D>
struct WT {
  using T = DT<FMT, D>;
  static constexpr int STAGE = 2 * T::STAGE;           // one 32-token step
  // copies per step of the waves that copy K codes, and of the others
  static constexpr int NK_DMA = (T::KB + 1023) / 1024;
  static constexpr int NR_DMA = (T::KSB + 1023) / 1024 + (T::VB + 1023) / 1024 + (T::VSB + 1023) / 1024;
  static constexpr bool VSH = T::VC != C_F16;          // V codes expanded into the shared buffer
  static constexpr int VSTEP = VSH ? 2 * D * 32 : 0;   // one step: [2 blocks][2 halves][D][8 tokens] f16
  static constexpr int BUDGET = 78 * 1024;             // two workgroups per CU
  // Where a ring of 3 stages fits beside two V buffers, step k + 1's V is
  // expanded during step k (one barrier per step); otherwise one buffer,
  // filled at the top of the step and published by a second barrier.
  static constexpr bool VDB = VSH && (BUDGET - 2 * VSTEP) / STAGE >= 3;
  static constexpr int VBUF = VDB ? 2 * VSTEP : VSTEP;
  static constexpr int FIT = (BUDGET - VBUF) / STAGE;
  static constexpr int S = FIT > 4 ? 4 : FIT;
  static_assert(S >= 2, "a step is read while the next one is in flight");
  static_assert(!VDB || S >= 3, "step k + 1 is expanded while step k + 2 is in flight");
  static constexpr int LDS = S * STAGE + VBUF;
  static constexpr int NT = D / 32;                    // 32-dim n-tiles of O^T
  static constexpr int KS = D / 16;                    // k-steps of Q.K
  static constexpr int KR = T::KBITS == 8 ? D / 32 : D / 16;  // 16-byte K reads per lane and step
};

// Four 16-byte LDS reads at addr + O0 .. O3, in one asm block that waits for
// them (the ring's copies stay in flight; see lds_read_part).
template <int O0, int O1, int O2, int O3>
__device__ __forceinline__ void lds_read4(uint4 (&r)[4], uint32_t addr) {
  asm volatile("ds_read_b128 %0, %4 offset:%5\n\tds_read_b128 %1, %4 offset:%6\n\t"
               "ds_read_b128 %2, %4 offset:%7\n\tds_read_b128 %3, %4 offset:%8\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
               : "v"(addr), "i"(O0), "i"(O1), "i"(O2), "i"(O3) : "memory");
}
template <int O0, int O1>
__device__ __forceinline__ void lds_read2(uint4 (&r)[2], uint32_t addr) {
  asm volatile("ds_read_b128 %0, %2 offset:%3\n\tds_read_b128 %1, %2 offset:%4\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(r[0]), "=&v"(r[1]) : "v"(addr), "i"(O0), "i"(O1) : "memory");
}
// Four 8-byte reads at addr + O0 .. O3.
template <int O0, int O1, int O2, int O3>
__device__ __forceinline__ void lds_read4x8(uint2 (&r)[4], uint32_t addr) {
  asm volatile("ds_read_b64 %0, %4 offset:%5\n\tds_read_b64 %1, %4 offset:%6\n\t"
               "ds_read_b64 %2, %4 offset:%7\n\tds_read_b64 %3, %4 offset:%8\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
               : "v"(addr), "i"(O0), "i"(O1), "i"(O2), "i"(O3) : "memory");
}
__device__ __forceinline__ uint2 lds_read8(uint32_t addr) {
  uint2 r;
  asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r) : "v"(addr) : "memory");
  return r;
}
__device__ __forceinline__ uint4 lds_read16(uint32_t addr) {
  uint4 r;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r) : "v"(addr) : "memory");
  return r;
}
__device__ __forceinline__ uint32_t lds_read4b(uint32_t addr) {
  uint32_t r;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r) : "v"(addr) : "memory");
  return r;
}
// Eight 8-byte writes at addr + 256 i, waiting for them.
__device__ __forceinline__ void lds_write8x8(uint32_t addr, const uint2 (&v)[8]) {
  asm volatile("ds_write_b64 %0, %1\n\tds_write_b64 %0, %2 offset:256\n\tds_write_b64 %0, %3 offset:512\n\t"
               "ds_write_b64 %0, %4 offset:768\n\tds_write_b64 %0, %5 offset:1024\n\t"
               "ds_write_b64 %0, %6 offset:1280\n\tds_write_b64 %0, %7 offset:1536\n\t"
               "ds_write_b64 %0, %8 offset:1792\n\ts_waitcnt lgkmcnt(0)"
               : : "v"(addr), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7])
               : "memory");
}
// Four 8-byte writes at addr + 256 i.
__device__ __forceinline__ void lds_write4x8(uint32_t addr, const uint2 (&v)[4]) {
  asm volatile("ds_write_b64 %0, %1\n\tds_write_b64 %0, %2 offset:256\n\tds_write_b64 %0, %3 offset:512\n\t"
               "ds_write_b64 %0, %4 offset:768\n\ts_waitcnt lgkmcnt(0)"
               : : "v"(addr), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]) : "memory");
}

__device__ __forceinline__ uint2 pack4(f16x2 a, f16x2 b) { return make_uint2(bitcast<uint32_t>(a), bitcast<uint32_t>(b)); }

// Expand the V codes of one 32-token step (stage at `stg`, first position
// t0) into the V^T buffer at `vbuf`, positions at or past L as zeros (slots
// past a sequence's end may hold any bytes).  All 256 threads take part.
template <int FMT, int D>
__device__ __forceinline__ void expand_v_step(uint32_t stg, uint32_t vbuf, int t0, int L, int tid) {
  using T = DT<FMT, D>;
  constexpr int G = T::VC == C_E4MX ? D / 32 : 1;
  if constexpr (T::VC == C_E2G16) {
    static_assert(D == 256, "4-bit V planes are built for head_dim 256");
    // thread (m, c, g, n): 16-byte chunk c of column n, tokens 4g..4g+3, of block m:
    // dims 16 (8c + jj) + n for jj < 8
    // (lane bit 0 and bit 5 give g, bits 1-4 give n: 16 lanes then write 128
    // consecutive bytes of the buffer, the two 8-byte halves of 8 slots)
    const int m = tid >> 7, c = (tid >> 6) & 1, g = (tid & 1) | ((tid >> 4) & 2), n = (tid >> 1) & 15;
    const uint32_t blk = stg + m * T::STAGE;
    const uint4 cw = lds_read16(blk + T::SV + c * 1024 + (16 * g + n) * 16);
    uint4 sw4[2];
    lds_read2<0, 16>(sw4, blk + T::SVS + g * 64 + 32 * c);
    const uint32_t sw[8] = {sw4[0].x, sw4[0].y, sw4[0].z, sw4[0].w, sw4[1].x, sw4[1].y, sw4[1].z, sw4[1].w};
    const uint32_t cws[4] = {cw.x, cw.y, cw.z, cw.w};
    const int p0 = t0 + 16 * m + 4 * g;  // position of token e = 0
    uint2 out[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const uint32_t w = cws[jj >> 1];
      f16x2 lo, hi;  // tokens 0, 1 and 2, 3
      if (jj & 1) {
        lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
        hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
      } else {
        lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
        hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
      }
      lo *= __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)sw[jj], 1.0f, false);
      hi *= __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)sw[jj], 1.0f, true);
      out[jj] = pack4(lo, hi);
    }
    if (p0 + 3 >= L) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        out[jj].x = p0 >= L ? 0u : (p0 + 1 >= L ? (out[jj].x & 0xFFFFu) : out[jj].x);
        out[jj].y = p0 + 2 >= L ? 0u : (p0 + 3 >= L ? (out[jj].y & 0xFFFFu) : out[jj].y);
      }
    }
    // dims 16 (8c + jj) + n, tokens 4g .. 4g + 3 = half g / 2, bytes 8 (g % 2) ..
    const uint32_t dst = vbuf + m * D * 32 + (g >> 1) * D * 16 + (128 * c + n) * 16 + (g & 1) * 8;
    lds_write8x8(dst, out);
  } else {
    // 8-bit codes: thread (m, c, g, n) per 16-byte chunk c of column n, tokens
    // 4g..4g+3, of block m: dims 16 (4c + jj) + n for jj < 4
    constexpr int NCH = D / 64;               // chunks per block
    constexpr int REPS = 2 * NCH * 64 / 256;  // chunks per thread
#pragma unroll
    for (int rep = 0; rep < REPS; ++rep) {
      const int ci = tid + 256 * rep;
      const int m = ci / (64 * NCH), c = (ci >> 6) % NCH, g = (ci & 1) | ((ci >> 4) & 2), n = (ci >> 1) & 15;
      const uint32_t blk = stg + m * T::STAGE;
      const uint4 cw = lds_read16(blk + T::SV + c * 1024 + (16 * g + n) * 16);
      const uint32_t cws[4] = {cw.x, cw.y, cw.z, cw.w};
      const int p0 = t0 + 16 * m + 4 * g;
      uint2 out[4];
      if constexpr (T::VC == C_E4MX) {
        // UE8M0 of (token 4g + e, group 2c + jj / 2): code x 2^e in fp32, one RNE to f16
        uint32_t sb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) sb[e] = lds_read4b(blk + T::SVS + (4 * g + e) * G + ((2 * c) & ~3)) >> (8 * ((2 * c) & 3));
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)cws[jj], false);
          const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)cws[jj], true);
          const float x[4] = {lo[0], lo[1], hi[0], hi[1]};
          f16x4 r;
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = (_Float16)ldexpf(x[e], (int)((sb[e] >> (8 * (jj >> 1))) & 0xFFu) - 127);
          out[jj] = bitcast<uint2>(r);
        }
      } else {
        uint2 s = make_uint2(0x3C003C00u, 0x3C003C00u);  // fp16 1.0 pairs
        if constexpr (T::VC == C_E4ROW) s = lds_read8(blk + T::SVS + 8 * g);  // fp16 scales of tokens 4g..4g+3
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)cws[jj], 1.0f, false);
          f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)cws[jj], 1.0f, true);
          if constexpr (T::VC == C_E4ROW) {
            lo *= bitcast<f16x2>(s.x);
            hi *= bitcast<f16x2>(s.y);
          }
          out[jj] = pack4(lo, hi);
        }
      }
      if (p0 + 3 >= L) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          out[jj].x = p0 >= L ? 0u : (p0 + 1 >= L ? (out[jj].x & 0xFFFFu) : out[jj].x);
          out[jj].y = p0 + 2 >= L ? 0u : (p0 + 3 >= L ? (out[jj].y & 0xFFFFu) : out[jj].y);
        }
      }
      const uint32_t dst = vbuf + m * D * 32 + (g >> 1) * D * 16 + (64 * c + n) * 16 + (g & 1) * 8;
      lds_write4x8(dst, out);
    }
  }
}

// 8 E4M3 codes -> bf16x8 times 2^(byte - 127) (the scaled conversion adds the
// exponent; exact while the result is a normal bf16).  Byte 0 is taken as 1.
__device__ __forceinline__ bf16x8 e4m3x8_bf16_mx(uint32_t w0, uint32_t w1, uint32_t byte) {
  const float sc = __uint_as_float((byte > 1u ? byte : 1u) << 23);
  uint4 r;
  r.x = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, sc, false));
  r.y = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, sc, true));
  r.z = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, sc, false));
  r.w = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, sc, true));
  return bitcast<bf16x8>(r);
}

template <int FMT, int D>
__global__ __launch_bounds__(256, 2) void prefill_wide_kernel(Geometry geo, DecodeArgs a, int tiles) {
  using T = DT<FMT, D>;
  using W = WT<FMT, D>;
  constexpr float NEG_INF = -__builtin_inff();
  extern __shared__ float lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, c32 = lane & 31;
  const int wi = blockIdx.x;  // item: 128 rows (a row tile) of one unit
  const int u = wi / tiles, tile = wi - u * tiles;
  const int b = u / geo.H_kv, h = u - b * geo.H_kv;
  const int L = as_const(a.seq_lens)[b];
  const uint32_t ring0 = (uint32_t)(uintptr_t)(void*)lds;
  const uint32_t vbuf = ring0 + W::S * W::STAGE;

  // ---- this wave's rows r0 .. r0 + 31; lane row c32 -> (query i, head)
  const int r0 = 128 * tile + 32 * wave;
  const bool has_rows = r0 < a.R;  // wave-uniform; a wave without rows still expands V and joins the barriers
  const int rr = r0 + c32;
  const bool row_ok = rr < a.R;
  const int qi = rr / a.G, qh = h * a.G + (rr - qi * a.G);
  const int limit = row_ok ? L - a.n_q + qi : -1;  // last visible position of the row
  const int wlim_lo = L - a.n_q + r0 / a.G;                            // the wave's first row
  const int wlim_hi = L - a.n_q + (min(a.R, r0 + 32) - 1) / a.G;       // and its last
  const int last_row = min(a.R, 128 * tile + 128) - 1;
  const int lim_wg = L - a.n_q + last_row / a.G;
  const int nk = lim_wg >= 0 ? (lim_wg >> 5) + 1 : 0;  // 32-token steps
  const int last_blk = lim_wg >> 4;

  // ---- Q^T operands: row c32, dims 16 ks + 8 hl .. + 7
  uint4 qv[W::KS];
  {
    const uint16_t* qp = a.q + (((int64_t)b * a.n_q + qi) * a.H_q + qh) * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < W::KS; ++ks) qv[ks] = row_ok ? *reinterpret_cast<const uint4*>(qp + 16 * ks) : make_uint4(0, 0, 0, 0);
  }
  // the K operand row of this lane: token tau = c32 with bits 2 and 3 swapped
  const int tau = (c32 & ~12) | ((c32 & 4) << 1) | ((c32 & 8) >> 1);
  const uint32_t koff = (tau >> 4) * T::STAGE + T::SK + (16 * hl + (tau & 15)) * 16;

  const uint8_t* head0 = a.pool + (int64_t)h * geo.head_bytes;
  const cint32* bt_row = as_const(a.block_table) + (int64_t)b * a.max_pages;
  // A step's copies are spread over the four waves: wave w takes token block
  // w % 2 of the step, its K codes (w < 2) or its K scales, V codes and V
  // scales (w >= 2); each wave waits for its own copies before the barrier
  // that publishes the step.
  auto stage_part = [&](int k, uint32_t dst) {
    const BlockAddr ba = block_addr(head0, geo, bt_row, (wave & 1) ? min(2 * k + 1, last_blk) : 2 * k);
    const uint32_t d = dst + (wave & 1) * T::STAGE;
    if (wave < 2) {
      copy_plane<T::KB, CPOL_REUSE>(d + T::SK, ba.hb + geo.off_kc + (int64_t)ba.bip * T::KB, lane);
    } else {
      if constexpr (T::KSB > 0)
        copy_plane<T::KSB, CPOL_REUSE>(d + T::SKS, ba.hb + geo.off_ks + (int64_t)ba.bip * T::KSB, lane);
      copy_plane<T::VB, CPOL_REUSE>(d + T::SV, ba.hb + geo.off_vc + (int64_t)ba.bip * T::VB, lane);
      if constexpr (T::VSB > 0)
        copy_plane<T::VSB, CPOL_REUSE>(d + T::SVS, ba.hb + geo.off_vs + (int64_t)ba.bip * T::VSB, lane);
    }
  };
  auto wait_part = [&](int after) {
    if (wave < 2) wait_staged<W::NK_DMA, W::S>(after);
    else wait_staged<W::NR_DMA, W::S>(after);
  };

  f32x16 O[W::NT];
#pragma unroll
  for (int nt = 0; nt < W::NT; ++nt)
#pragma unroll
    for (int j = 0; j < 16; ++j) O[nt][j] = 0.f;
  float m_run = NEG_INF, l_run = 0.f;

  constexpr int S = W::S;
#pragma unroll
  for (int k = 0; k < S - 1; ++k)
    if (k < nk) stage_part(k, ring0 + k * W::STAGE);
  if constexpr (W::VDB) {
    if (nk > 0) {
      wait_part(min(S - 2, nk - 1));
      __syncthreads();
      expand_v_step<FMT, D>(ring0, vbuf, 0, L, tid);
    }
  }
  int st = 0;
  for (int k = 0; k < nk; ++k) {
    // With two V buffers the waves wait for step k + 1 (k landed before), else for step k.
    if constexpr (W::VDB) {
      if (k + 1 < nk) wait_part(min(S - 3, nk - 2 - k));
    } else {
      wait_part(min(S - 2, nk - 1 - k));
    }
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();  // the step(s) landed; every wave is done with step k - 1 (its stage and V buffer)
    if (k + S - 1 < nk) stage_part(k + S - 1, ring0 + ((st + S - 1) % S) * W::STAGE);
    const uint32_t stg = ring0 + st * W::STAGE;
    const int st1 = st + 1 == S ? 0 : st + 1;
    const int t0 = 32 * k;
    uint32_t vcur = vbuf;  // the V buffer of step k
    if constexpr (W::VDB) {
      vcur = vbuf + (k & 1) * W::VSTEP;
      if (k + 1 < nk) expand_v_step<FMT, D>(ring0 + st1 * W::STAGE, vbuf + ((k + 1) & 1) * W::VSTEP, t0 + 32, L, tid);
    } else if constexpr (W::VSH) {
      expand_v_step<FMT, D>(stg, vbuf, t0, L, tid);
    }
    st = st1;

    const bool active = has_rows && t0 <= wlim_hi;  // wave-uniform: some row sees a token of this step
    f16x8 P0, P1;
    if (active) {
      // the products run at raised priority, the softmax and the expansion
      // at the base one, so a SIMD's matrix core is fed first
      __builtin_amdgcn_s_setprio(1);
      // ---- S^T = K Q^T (rows: tokens tau, columns: the wave's rows)
      f32x16 Sacc;
#pragma unroll
      for (int j = 0; j < 16; ++j) Sacc[j] = 0.f;
      uint32_t mxs[2] = {0u, 0u};  // MXFP8: the UE8M0 of the lane's token, group ks / 2 in byte ks / 2
      if constexpr (T::KC == C_E4MX) {
        const uint32_t sa = stg + (tau >> 4) * T::STAGE + T::SKS + (tau & 15) * (D / 32);
        if constexpr (D == 256) {
          const uint2 s2 = lds_read8(sa);
          mxs[0] = s2.x; mxs[1] = s2.y;
        } else {
          mxs[0] = lds_read4b(sa);
        }
      }
#pragma unroll
      for (int bt = 0; bt < W::KR / 4; ++bt) {
        uint4 kr[4];
        lds_read4<0, 512, 1024, 1536>(kr, stg + koff + bt * 2048);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (T::KBITS == 16) {
            Sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(kr[i]), bitcast<bf16x8>(qv[4 * bt + i]), Sacc, 0, 0, 0);
          } else {
            // read 2 a + b (a = 2 bt + i / 2, b = i % 2) holds k-step 4 a + b (bytes 0-7) and 4 a + 2 + b
            const int ka = 4 * (2 * bt + (i >> 1)) + (i & 1), kb = ka + 2;
            bf16x8 x0, x1;
            if constexpr (T::KC == C_E4MX) {
              x0 = e4m3x8_bf16_mx(kr[i].x, kr[i].y, (mxs[(ka >> 1) >> 2] >> (8 * ((ka >> 1) & 3))) & 0xFFu);
              x1 = e4m3x8_bf16_mx(kr[i].z, kr[i].w, (mxs[(kb >> 1) >> 2] >> (8 * ((kb >> 1) & 3))) & 0xFFu);
            } else {
              x0 = e4m3x8_bf16(kr[i].x, kr[i].y);
              x1 = e4m3x8_bf16(kr[i].z, kr[i].w);
            }
            Sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x0, bitcast<bf16x8>(qv[ka]), Sacc, 0, 0, 0);
            Sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x1, bitcast<bf16x8>(qv[kb]), Sacc, 0, 0, 0);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // ---- scores in log2 units, causal limit (positions past L included)
      float sc[16];
      if constexpr (T::KC == C_E4ROW) {
        // fp16 row scales of tokens 16 m + 8 hl .. + 7
        uint4 ks2[2];
        lds_read2<0, T::STAGE>(ks2, stg + T::SKS + 16 * hl);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint32_t w4[4] = {ks2[m].x, ks2[m].y, ks2[m].z, ks2[m].w};
#pragma unroll
          for (int i = 0; i < 8; ++i)
            sc[8 * m + i] = Sacc[8 * m + i] * (a.qk_scale * f16_bits_to_f32((w4[i >> 1] >> (16 * (i & 1))) & 0xFFFFu));
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) sc[j] = Sacc[j] * a.qk_scale;
      }
      if (t0 + 31 > wlim_lo) {  // wave-uniform: some row of the wave stops inside this step
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (t0 + 16 * (j >> 3) + 8 * hl + (j & 7) > limit) sc[j] = NEG_INF;
      }
      // ---- online softmax with the lazy running maximum (the decode kernel's rule)
      float bm = sc[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) bm = fmaxf(bm, sc[j]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(bitcast<uint32_t>(bm), bitcast<uint32_t>(bm), false, false);
        bm = fmaxf(bitcast<float>((uint32_t)sw[0]), bitcast<float>((uint32_t)sw[1]));
      }
      if (__any(bm > m_run + RESCALE_SLACK)) {
        const float m_new = fmaxf(m_run, bm);
        const float corr = (m_new > m_run) ? fast_exp2(m_run - m_new) : 1.0f;
        l_run *= corr;
#pragma unroll
        for (int nt = 0; nt < W::NT; ++nt)
#pragma unroll
          for (int j = 0; j < 16; ++j) O[nt][j] *= corr;
        m_run = m_new;
      }
      const float m_use = (m_run == NEG_INF) ? 0.f : m_run;
      float p[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        p[j] = fast_exp2(sc[j] - m_use);
        l_run += p[j];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        P0[i] = (_Float16)p[i];
        P1[i] = (_Float16)p[8 + i];
      }
    }
    if constexpr (W::VSH && !W::VDB) __syncthreads();  // the V buffer is complete
    if (active) {
      __builtin_amdgcn_s_setprio(1);
      // ---- O^T += V^T P^T, two 16-token products per 32-dim n-tile
      if constexpr (W::VSH) {
        const uint32_t vb = vcur + hl * D * 16 + c32 * 16;
#pragma unroll
        for (int nt = 0; nt < W::NT; nt += 2) {
          uint4 v4[4];
          lds_read4<0, D * 32, 512, 512 + D * 32>(v4, vb + nt * 512);
          O[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<f16x8>(v4[0]), P0, O[nt], 0, 0, 0);
          O[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<f16x8>(v4[1]), P1, O[nt], 0, 0, 0);
          O[nt + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<f16x8>(v4[2]), P0, O[nt + 1], 0, 0, 0);
          O[nt + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<f16x8>(v4[3]), P1, O[nt + 1], 0, 0, 0);
        }
      } else {
        // fp16 V straight from the stage: dim 32 nt + c32 = 16 jt + n, jt = 2 nt + c32 / 16;
        // tokens 8 hl + i: slab rows g = 2 hl (i < 4) and 2 hl + 1, 4 tokens (8 bytes) each
        const uint32_t vb = stg + T::SV + (32 * hl + (c32 & 15)) * 16 + (c32 >> 4) * 8;
        const bool tail = t0 + 31 >= L;  // wave-uniform
#pragma unroll
        for (int nt = 0; nt < W::NT; ++nt) {
          uint2 v2[4];
          lds_read4x8<0, 256, T::STAGE, T::STAGE + 256>(v2, vb + nt * 1024);
          f16x8 va = bitcast<f16x8>(make_uint4(v2[0].x, v2[0].y, v2[1].x, v2[1].y));
          f16x8 vc = bitcast<f16x8>(make_uint4(v2[2].x, v2[2].y, v2[3].x, v2[3].y));
          if (tail) {  // positions at or past L may hold any bits
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              if (t0 + 8 * hl + i >= L) va[i] = (_Float16)0.f;
              if (t0 + 16 + 8 * hl + i >= L) vc[i] = (_Float16)0.f;
            }
          }
          O[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, P0, O[nt], 0, 0, 0);
          O[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vc, P1, O[nt], 0, 0, 0);
        }
      }
    }
  }
  if (!has_rows) return;

  // ---- finish the rows: l over the lane pair; O^T register j of n-tile nt
  // holds dim 32 nt + 8 (j / 4) + 4 hl + j % 4 of row c32
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(bitcast<uint32_t>(l_run), bitcast<uint32_t>(l_run), false, false);
    l_run = bitcast<float>((uint32_t)sw[0]) + bitcast<float>((uint32_t)sw[1]);
  }
  const float inv = l_run > 0.f ? a.v_out_scale / l_run : 0.f;
#pragma unroll
  for (int nt = 0; nt < W::NT; ++nt)
#pragma unroll
    for (int j = 0; j < 16; ++j) O[nt][j] *= inv;
  if constexpr (T::VROT) {
    // o = H o' / 16: the lane's 128 values are indexed by dim bits 0-1, 3-7
    // (f = 16 nt + j), bit 2 is the lane pair
    static_assert(D == 256, "the rotation is 256-point");
#pragma unroll
    for (int hb = 1; hb < 128; hb <<= 1)
#pragma unroll
      for (int f = 0; f < 128; ++f)
        if ((f & hb) == 0) {
          const float x = O[f >> 4][f & 15], y = O[(f + hb) >> 4][(f + hb) & 15];
          O[f >> 4][f & 15] = x + y;
          O[(f + hb) >> 4][(f + hb) & 15] = x - y;
        }
#pragma unroll
    for (int nt = 0; nt < W::NT; ++nt)
#pragma unroll
      for (int j = 0; j < 16; ++j) O[nt][j] = xlane_butterfly<32>(O[nt][j], lane) * 0.0625f;
  }
  if (row_ok) {
    float* op = a.out + (((int64_t)b * a.n_q + qi) * a.H_q + qh) * D + 4 * hl;
#pragma unroll
    for (int nt = 0; nt < W::NT; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(op + 32 * nt + 8 * q) =
            make_float4(O[nt][4 * q], O[nt][4 * q + 1], O[nt][4 * q + 2], O[nt][4 * q + 3]);
    if (a.lse != nullptr && hl == 0)
      a.lse[((int64_t)b * a.n_q + qi) * a.H_q + qh] =
          l_run > 0.f ? (m_run + __log2f(l_run)) * 0.69314718055994531f : NEG_INF;
  }
}

template <int FMT, int D>
hipError_t launch_prefill_t(const Geometry& geo, const DecodeArgs& a, hipStream_t stream) {
  if constexpr (wide_prefill_format<FMT>()) {
    const int64_t tiles = (a.R + 127) / 128;
    const int64_t total = (int64_t)a.B * geo.H_kv * tiles;
    if (total == 0) return hipSuccess;
    constexpr size_t lds = WT<FMT, D>::LDS;
    hipLaunchKernelGGL((prefill_wide_kernel<FMT, D>), dim3((unsigned)total), dim3(256), lds, stream, geo, a,
                       (int)tiles);
  } else {
    const int64_t tiles = (a.R + 63) / 64;
    const int64_t total = (int64_t)a.B * geo.H_kv * tiles;
    if (total == 0) return hipSuccess;
    constexpr size_t lds = prefill_lds_bytes<FMT, D>();
    hipLaunchKernelGGL((prefill_kernel<FMT, D>), dim3((unsigned)total), dim3(256), lds, stream, geo, a, (int)tiles);
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const Geometry& geo, const DecodeArgs& a, hipStream_t stream) {
#define KVQ_PREFILL_CASE(F, DD) \
  if (geo.fmt == F && geo.D == DD) return launch_prefill_t<F, DD>(geo, a, stream);
  KVQ_FOR_EACH_DECODE(KVQ_PREFILL_CASE)
#undef KVQ_PREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
