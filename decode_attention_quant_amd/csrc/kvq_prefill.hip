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
// with the lazy running maximum, P.V).  The work items are laid out so that
// one unit's row tiles run on one XCD, whose L2 then serves the repeats, so
// HBM sees a unit's cache about once per XCD.  Each wave finishes its own
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

// One work item = 64 rows (a row tile) of one unit; item wi runs on workgroup
// n with wi = (n % 8) * chunk + n / 8, so the items of one unit, which are
// consecutive, share an XCD (workgroups go to the 8 XCDs round robin).
template <int FMT, int D>
__global__ __launch_bounds__(256, 2) void prefill_kernel(Geometry geo, DecodeArgs a, int tiles, int chunk) {
  using T = DT<FMT, D>;
  using PP = PT<FMT, D>;
  constexpr float NEG_INF = -__builtin_inff();
  constexpr int E = D / 64;
  extern __shared__ float lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int n = blockIdx.x;
  const int wi = (n & 7) * chunk + (n >> 3);
  if (wi >= a.B * geo.H_kv * tiles) return;
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

hipError_t launch_prefill(const Geometry& geo, const DecodeArgs& a, hipStream_t stream) {
  const int64_t tiles = (a.R + 63) / 64;
  const int64_t total = (int64_t)a.B * geo.H_kv * tiles;
  if (total == 0) return hipSuccess;
  const int64_t chunk = (total + 7) / 8;
#define KVQ_PREFILL_CASE(F, DD)                                                                       \
  if (geo.fmt == F && geo.D == DD) {                                                                  \
    const size_t lds = prefill_lds_bytes<F, DD>();                                                    \
    hipLaunchKernelGGL((prefill_kernel<F, DD>), dim3((unsigned)(8 * chunk)), dim3(256), lds, stream, \
                       geo, a, (int)tiles, (int)chunk);                                               \
    return hipGetLastError();                                                                         \
  }
  KVQ_FOR_EACH_DECODE(KVQ_PREFILL_CASE)
#undef KVQ_PREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
