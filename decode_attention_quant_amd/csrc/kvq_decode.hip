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
// (x, row tile) takes an equal slice of it, counting a fixed cost for each
// further unit a slice reaches into, so every workgroup streams about the
// same number of bytes whatever the length mix.  A
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
//     MXFP4 (K)       E2M1 x 2^e -> f16 by the scaled conversion (exact) x
//                     rotated q as f16 hi + lo
//     MXFP8, query-MXFP8 mode: E4M3 K x E4M3 q on the block-scaled fp8
//                     MFMA, both UE8M0 scales applied by the instruction
//   online softmax in base 2, masking t >= L and the MTP causal rule;
//   O (16 rows x D) += P . V_blk (16x16x16 f16), P rounded to f16 and V
//   expanded to f16 with its scale folded in: exact for fp16 V and for
//   E2M1 x UE4M3; one f16 rounding of code x scale for int8 and E4M3 with
//   an fp16 scale and for E4M3 x 2^e; the per-tensor V scale (and the
//   second level of two-level NVFP4) multiplies the output instead.
//
// Blocks reach a wave through its ring of LDS stages (direct global -> LDS
// copies, S - 1 blocks in flight), except BF16 at head_dim 256, whose
// blocks do not fit and go through registers.
#include <hip/hip_runtime.h>

#include "kvq_decode_core.hpp"
#include "kvq_encode.hpp"

namespace kvq {

// ----------------------------------------------------------- fused append

// The new tokens of sequence b, kv head h at positions [plo, phi) (at most
// one 16-token block; input token i of sequence b is row b * n_q + i of
// k_new / v_new) are encoded one token at a time by the whole wave, with the
// write path's single-token encoders, so the bytes are those quantize-append
// stores.  The raw rows of the first TB tokens are loaded at the segment's
// start, so that their latency overlaps the query's and the first blocks'.
template <int D>
struct NewRows {
  static constexpr int TB = D == 256 ? 2 : 4;
  enc::TokenRow<D> k[TB], v[TB];
};

__device__ __forceinline__ int64_t new_row(const DecodeArgs& a, const Geometry& geo, int b, int h, int i) {
  return (((int64_t)b * a.n_q + i) * geo.H_kv + h) * geo.D;
}

template <int D>
__device__ __forceinline__ void load_new_rows(NewRows<D>& nr, const DecodeArgs& a, const Geometry& geo, int b, int h,
                                              int L, int plo, int phi, int lane) {
  const int ilo = plo - (L - a.n_q), ihi = phi - (L - a.n_q);
#pragma unroll
  for (int u = 0; u < NewRows<D>::TB; ++u) {
    const int64_t row = new_row(a, geo, b, h, min(ilo + u, ihi - 1));  // issued on every path
    enc::load_k_token<D>(nr.k[u], a.k_new + row, lane);
    enc::load_v_token<D>(nr.v[u], a.v_new + row, lane);
  }
}

template <int FMT, int D>
__device__ __forceinline__ void store_new_tokens(const NewRows<D>& nr, const DecodeArgs& a, const Geometry& geo, int b,
                                                 int h, int L, int plo, int phi, int lane) {
  const int pnew = L - a.n_q;  // position of new token 0
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  auto slot_at = [&](int p) -> int { return bt[p / geo.P] * geo.P + p % geo.P; };
  auto put = [&](const enc::TokenRow<D>& rk, const enc::TokenRow<D>& rv, int p) {
    const int slot = slot_at(p);
    enc::encode_k_token<base_format(FMT), D>(a.pool_w, rk, slot, geo, h, a.enc_k_scale, lane);
    enc::encode_v_token<base_format(FMT), D>(a.pool_w, rv, slot, geo, h, a.enc_v_scale, lane);
  };
#pragma unroll
  for (int u = 0; u < NewRows<D>::TB; ++u)
    if (plo + u < phi) put(nr.k[u], nr.v[u], plo + u);
  for (int p = plo + NewRows<D>::TB; p < phi; ++p) {
    enc::TokenRow<D> rk, rv;
    const int64_t row = new_row(a, geo, b, h, p - pnew);
    enc::load_k_token<D>(rk, a.k_new + row, lane);
    enc::load_v_token<D>(rv, a.v_new + row, lane);
    put(rk, rv, p);
  }
}

// ----------------------------------------------------------- the kernel

// The split ranges.  The blocks of all units u = b * H_kv + h in order,
// with c = DecodeArgs::seg_cost more between one unit and the next, form a
// line of C = T + c (units - 1) cost positions: a workgroup pays a
// segment's start-up and merge again for each further unit it visits, so
// one whose range crosses into the next unit takes about c blocks fewer.
// Block i of unit (b, h) sits at cost cum[b] + h * nb + c * (b * H_kv + h)
// + i.  Workgroup w of the `ways` that get work holds the costs
// [floor(w C / ways), floor((w + 1) C / ways)): exact shares, so that ranges
// that would line up with the units (c = 0, equal units) still do, the
// drift staying inside the c positions between two units.

// Workgroups that get work: all of them, unless that leaves fewer than
// clamp(C / 256, 4, 128) positions each (sequences much shorter than the
// grid was sized for): then at most 256 longer ranges, and the rest empty.
// The floor of 4 blocks is one per wave: at 1 x 1024 tokens (128 blocks) a
// floor of 16 made each wave stream 4 blocks one after another, and the
// split took 12.4 us instead of 8.7.
__host__ __device__ __forceinline__ int split_ways(int64_t C, int nwg) {
  int64_t lo = (C + 255) / 256;
  lo = lo < 4 ? 4 : (lo > 128 ? 128 : lo);
  const int64_t ways = (C + lo - 1) / lo;
  return ways < 1 ? 1 : (ways < nwg ? (int)ways : nwg);
}

// The first cost position of workgroup w (C for w >= ways).
__host__ __device__ __forceinline__ int64_t split_range_start(int64_t C, int ways, int w) {
  return w >= ways ? C : (int64_t)w * C / ways;
}

// The workgroup that holds cost position y (0 <= y < C).
__host__ __device__ __forceinline__ int split_range_of(int64_t C, int ways, int64_t y) {
  return (int)(((y + 1) * ways - 1) / C);
}

// The blocks at cost positions below y (cum: the prefix table in LDS).
__device__ __forceinline__ int blocks_before_cost(const int* cum, const int32_t* seq_lens, int B, int H_kv, int c,
                                                  int64_t y) {
  // with c positions before every unit, unit 0's too, unit (b, h) spans
  // [s, s + c + nb), s = cum[b] + c * H_kv * b + h * (nb + c)
  y += c;
  const int64_t cb = (int64_t)c * H_kv;
  if (y >= cum[B] + cb * B) return cum[B];
  int lo = 0, hi = B;  // cost(lo) <= y < cost(hi), cost(b) = cum[b] + c * H_kv * b
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cum[mid] + cb * mid <= y) lo = mid; else hi = mid;
  }
  const int nb = (as_const(seq_lens)[lo] + 15) >> 4;  // nb + c > 0: sequence lo spans y
  const int r = (int)(y - (cum[lo] + cb * lo));
  const int h = r / (nb + c);
  const int off = r - h * (nb + c) - c;
  return cum[lo] + h * nb + (off > 0 ? off : 0);
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
    int run = 0, first = 0;  // first: blocks of sequence b0 (the only one when B <= 256)
    for (int i = 0; i < per_t; ++i) {
      const int bb = b0 + i;
      if (bb < a.B) {
        const int nbk = ((a.seq_lens[bb] + 15) >> 4) * geo.H_kv;
        if (i == 0) first = nbk;
        run += nbk;
      }
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
        base += i == 0 ? first : ((a.seq_lens[bb] + 15) >> 4) * geo.H_kv;
      }
    }
    if (threadIdx.x == 0) cum[a.B] = __float_as_int(tot[256]);
    __syncthreads();
  }
  const int total = cum[a.B];
  if (w == 0 && rt == 0)
    for (int i = threadIdx.x; i <= a.B; i += 256) a.ws_cum[i] = cum[i];
  const int units = a.B * geo.H_kv;
  const int64_t C = total + (int64_t)a.seg_cost * (units > 1 ? units - 1 : 0);
  const int ways = split_ways(C, a.nwg);
  int x = blocks_before_cost(cum, a.seq_lens, a.B, geo.H_kv, a.seg_cost, split_range_start(C, ways, w));
  const int x_end = blocks_before_cost(cum, a.seq_lens, a.B, geo.H_kv, a.seg_cost, split_range_start(C, ways, w + 1));

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
    // A segment's start-up is a chain of latencies (the query, the first
    // copies, the new tokens' stores): it runs at the top priority, ahead of
    // the other workgroup's waves streaming on the same SIMDs.
    __builtin_amdgcn_s_setprio(3);

    // ---- fused step: the wave that owns a block holding new tokens stores
    //      them (n_q <= 16: at most two blocks, so two waves).  Only that
    //      wave reads the block (one row tile, one owner), through the same
    //      L2, so its stores and atomics only have to be complete before its
    //      own copy of the block is issued; the atomics of 4-bit V codes
    //      touch only cache lines of the block's own code plane.  Loads and
    //      stores of a wave complete in order as far as the vector-memory
    //      counter goes, so a ring block staged at iteration k >= 1, issued
    //      after the wait for block k - 1, needs no wait of its own.  The new
    //      rows are loaded here, so that they arrive with the query.  A block
    //      staged at start-up is stored first and waited for; a block that
    //      the ring stages later is stored just before the block loop.
    int kmine = -1;  // this wave's index k of its block with new tokens
    int mlo = 0, mhi = 0;
    if constexpr (FUSED) {
      const int plo = max(max(L - a.n_q, 0), 16 * blk0), phi = min(L, 16 * (blk0 + nblk));
      for (int jb = plo >> 4; plo < phi && jb <= (phi - 1) >> 4; ++jb) {
        if (((jb - blk0) & 3) == wave) {
          kmine = (jb - blk0) >> 2;
          mlo = max(plo, 16 * jb);
          mhi = min(phi, 16 * jb + 16);
        }
      }
    }
    const bool late_append = T::RING && kmine >= T::RING_S - 1;
    NewRows<D> nr;
    if (FUSED && kmine >= 0) load_new_rows<D>(nr, a, geo, b, h, L, mlo, mhi, lane);
    if (FUSED && kmine >= 0 && !late_append) {
      store_new_tokens<FMT, D>(nr, a, geo, b, h, L, mlo, mhi, lane);
      wait_vmcnt<0>();
    }

    // ---- query rows of this tile: row r (= c16 in S layout) -> (i, head)
    const int r = c16;
    const int rr = 16 * rt + r;
    const bool row_ok = r < Rt;
    const int qi = rr / a.G, qh = h * a.G + (rr - qi * a.G);
    const int limit = row_ok ? L - a.n_q + qi : -1;  // last visible position of this row
    float crow = a.qk_scale;
    const uint8_t* head0 = a.pool + (int64_t)h * geo.head_bytes;
    const cint32* bt_row = as_const(a.block_table) + (int64_t)b * a.max_pages;

    // ---- start-up latencies overlap: the page numbers of this wave's first
    //      blocks and the query rows are loaded together, and the first
    //      blocks' copies go out before the query setup (for a rotated query
    //      on a ring, only the first block's: the others would stall the
    //      wave while the memory queues are full, so they follow the setup)
    //      All of these loads are issued on every path (indexes past the end
    //      are clamped to valid ones, whose data is then not used), so that
    //      the compiler can count them exactly and does not drain every
    //      outstanding load where paths join.
    int nk = 0;  // ring formats: this wave's blocks blk0 + wave + 4 k, k < nk
    BlockAddr pre[T::RING ? T::RING_S - 1 : 1];
    if constexpr (T::RING) {
      nk = nblk > wave ? (nblk - wave + 3) >> 2 : 0;
#pragma unroll
      for (int k = 0; k < T::RING_S - 1; ++k)
        pre[k] = block_addr(head0, geo, bt_row, min(blk0 + wave + 4 * k, blk0 + nblk - 1));
    }
    // copies of this wave's blocks k0 .. k1 - 1 (blocks k >= nk land in
    // stages that are never read)
    auto stage_first = [&](int k0, int k1) {
      if constexpr (T::RING) {
#pragma unroll
        for (int k = 0; k < T::RING_S - 1; ++k)
          if (k >= k0 && k < k1) stage_block_at<FMT, D>(ring0 + k * T::STAGE, pre[k], geo, lane);
      }
    };
    QOps<FMT, D> qo;
    qo.lane = lane;
    qo.lds = qst;
    uint4 qv[T::QSTEPS * T::QPIECES];
    constexpr int E = D / 64;
    if constexpr (T::QMX) {
      // q rounded to MXFP8 in the block-scaled MFMA's lane order (see
      // lds_read_qmx): for MFMA s, lane (g, r) holds d = 128 s + 16 g + [0, 16)
      // (half 0: MX group 4 s + g / 2) and d = 128 s + 64 + 16 g + [0, 16)
      // (half 1: group 4 s + 2 + g / 2); the other 16 values of both groups
      // are in lane (g ^ 1, r).
      const uint16_t* qp = a.q + (((int64_t)b * a.n_q + qi) * a.H_q + qh) * D;
      uint4 qraw[4 * T::QSTEPS];
#pragma unroll
      for (int i = 0; i < 4 * T::QSTEPS; ++i) {
        uint4 q4 = make_uint4(0, 0, 0, 0);
        if (row_ok) q4 = *reinterpret_cast<const uint4*>(qp + 128 * (i >> 2) + 64 * ((i >> 1) & 1) + 16 * g + 8 * (i & 1));
        qraw[i] = q4;
      }
      stage_first(0, T::RING_S - 1);
#pragma unroll
      for (int s = 0; s < T::QSTEPS; ++s) {
        uint32_t sb[2], w[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float x[16];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const uint4 v = qraw[4 * s + 2 * hh + u];
            const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              x[8 * u + 2 * j] = bf16_to_f32(vw[j] & 0xFFFFu);
              x[8 * u + 2 * j + 1] = bf16_to_f32(vw[j] >> 16);
            }
          }
          float am = 0.f;
#pragma unroll
          for (int j = 0; j < 16; ++j) am = fmaxf(am, fabsf(x[j]));
          am = fmaxf(am, __shfl_xor(am, 16));  // the group's other half
          float unused_s, unused_r;
          enc::group_scale<C_E4MX>(am, unused_s, unused_r, sb[hh]);
#pragma unroll
          for (int j = 0; j < 16; j += 4) {
            const int sh = 127 - (int)sb[hh];
            const uint32_t lo = enc::e4m3_pair<false>(0u, ldexpf(x[j], sh), ldexpf(x[j + 1], sh));
            w[4 * hh + j / 4] = enc::e4m3_pair<true>(lo, ldexpf(x[j + 2], sh), ldexpf(x[j + 3], sh));
          }
        }
        qv[2 * s] = make_uint4(w[0], w[1], w[2], w[3]);
        qv[2 * s + 1] = make_uint4(w[4], w[5], w[6], w[7]);
        // lane block g gives the scale of group 4 s + g: blocks 0 and 3 hold
        // it (half 0, half 1), blocks 1 and 2 hold each other's
        const uint32_t send = g == 2 ? sb[0] : sb[1];
        const uint32_t got = (uint32_t)__shfl((int)send, g == 1 ? lane + 16 : g == 2 ? lane - 16 : lane);
        qo.qsc[s] = g == 0 ? sb[0] : g == 3 ? sb[1] : got;
      }
    } else if constexpr (!T::QROT) {
      const uint16_t* qp = a.q + (((int64_t)b * a.n_q + qi) * a.H_q + qh) * D;
#pragma unroll
      for (int kk = 0; kk < T::QSTEPS; ++kk) {
        uint4 q4 = make_uint4(0, 0, 0, 0);
        if (row_ok) q4 = *reinterpret_cast<const uint4*>(qp + 32 * kk + 8 * g);
        qv[kk] = q4;
      }
      stage_first(0, T::RING_S - 1);
      // Take the query operands here, not at their first use inside the
      // block loop: a register load still pending at the loop entry makes
      // the compiler wait for every load (vmcnt 0) in each iteration, which
      // would drain the ring.
#pragma unroll
      for (int i = 0; i < T::QSTEPS; ++i) asm volatile("" : : "v"(qv[i].x), "v"(qv[i].y), "v"(qv[i].z), "v"(qv[i].w));
    } else {
      // q' = H q / 16 in fp32 for rows wave, wave + 4, ... of the tile,
      // transposed through LDS: for ring formats row `row` sits in the last
      // stage of wave (row & 3)'s ring, which no copy targets before the
      // block loop, and is written and read with the self-waiting accesses
      // above while the first blocks are in flight; otherwise row `row` of
      // the merge area.  max|q'| of row `row` goes to qexp[row].
      static_assert(E == 4, "the rotation is 256-point");
      auto qrow_ptr = [&](int i) -> const uint16_t* {
        const int row = wave + 4 * i < Rt ? wave + 4 * i : 0;  // rows past Rt load row 0, unused
        const int rr2 = 16 * rt + row;
        const int i2 = rr2 / a.G, h2 = h * a.G + (rr2 - i2 * a.G);
        return a.q + (((int64_t)b * a.n_q + i2) * a.H_q + h2) * D;
      };
      uint2 qraw[4];
      if constexpr (T::RING) {
        // The raw rows come in by the same direct copies as the blocks, into
        // the last stage of this wave's ring (row wave + 4 i at byte 512 i,
        // two rows per copy); a register load would make the compiler wait
        // for every copy issued after it before its first use.  The first
        // block's copies go out once the rows have landed: issued together,
        // the rows queue behind every wave's block copies (measured 5%
        // slower at 8 x 64K tokens), while the block is not needed before
        // the query setup ends anyway.
        const uint32_t qstage = ring0 + (T::RING_S - 1) * T::STAGE;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          __builtin_amdgcn_global_load_lds((gbl_void_t*)(qrow_ptr(2 * j + (lane >> 5)) + 8 * (lane & 31)),
                                           (lds_void_t*)(uintptr_t)(qstage + 1024 * j), 16, 0, CPOL_STREAM);
        wait_vmcnt<0>();
        stage_first(0, 1);
        lds_get_rows4(qstage + 8 * lane, qraw);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) qraw[i] = *reinterpret_cast<const uint2*>(qrow_ptr(i) + E * lane);
      }
      // rows past Rt are neither transformed nor written: the lanes that
      // would read them select 0 instead (qrow_ok below)
      float xq[4][E], amx[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (wave + 4 * i < Rt) {
          xq[i][0] = bf16_to_f32(qraw[i].x & 0xFFFFu); xq[i][1] = bf16_to_f32(qraw[i].x >> 16);
          xq[i][2] = bf16_to_f32(qraw[i].y & 0xFFFFu); xq[i][3] = bf16_to_f32(qraw[i].y >> 16);
          fwht_wave<E>(xq[i], lane);
          float am = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) { xq[i][e] *= 0.0625f; am = fmaxf(am, fabsf(xq[i][e])); }
          am = wave_max(am);
          amx[i] = am;
        }
      }
      const uint32_t qexp_a = (uint32_t)(uintptr_t)(void*)qexp;
      // LDS byte address of row `row` (ring formats).  The rings' strides
      // are multiples of 256 bytes, so rows placed 1 KB apart would put the
      // 16 lanes that read 16 different rows at one offset into one bank;
      // row r is shifted by 16 r bytes, and those lanes read 16 distinct
      // 16-byte slots of every 256.
      auto qrow_a = [&](int row) -> uint32_t {
        return (uint32_t)(uintptr_t)(void*)sm_o +
               (uint32_t)((row & 3) * T::RING_S * T::STAGE + (T::RING_S - 1) * T::STAGE + (row >> 2) * D * 4 +
                          16 * row);
      };
      if constexpr (T::RING) static_assert(T::STAGE >= 4 * D * 4 + 16 * 15, "four shifted rows fit a stage");
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wave + 4 * i;
        if (row < Rt) {
          if constexpr (T::RING) {
            lds_put4(qrow_a(row) + 16 * lane, xq[i][0], xq[i][1], xq[i][2], xq[i][3]);
            if (lane == 0) lds_put1(qexp_a + 4 * row, amx[i]);
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) sm_o[row * D + E * lane + e] = xq[i][e];
            if (lane == 0) qexp[row] = amx[i];
          }
        }
      }
      // The rows are in LDS once each write has waited for itself; a bare
      // barrier then publishes them (__syncthreads' fence would also wait
      // for the copies in flight).
      if constexpr (T::RING) __builtin_amdgcn_s_barrier();
      else __syncthreads();
      // 8 consecutive elements d0 .. d0 + 7 of this lane's row r
      // xr[k][e] = element 32 k + 8 g + e of this lane's row r (all at once).
      // Packed (at most 8 rows): lanes c16 and c16 + 8 both take row c16 % 8;
      // the first gives the query's first piece, the second its second.
      const int qr = T::PACK ? (c16 & 7) : r;
      const bool qrow_ok = qr < Rt;
      float xr[8][8];
      if constexpr (T::RING) {
        lds_get_8x8(qrow_a(qr) + 32 * g, xr);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
          for (int e = 0; e < 8; ++e) xr[k][e] = sm_o[qr * D + 32 * k + 8 * g + e];
      }
      float am = 0.f;
      if (qrow_ok) {
        if constexpr (T::RING) am = lds_get1(qexp_a + 4 * qr);
        else am = qexp[qr];
      }
      const bool second_piece = T::PACK && (c16 & 8) != 0;
      if constexpr (T::QI8) {
        // q' ~ (c1 + c2 / 254) / inv, int8 c1 = RN(q' inv), c2 = RN(254 (q' inv - c1)),
        // inv = 127 / max|q'|: error below max|q'| / 64516 per element
        const float inv = am > 0.f ? 127.0f / am : 0.f;
        crow = am > 0.f ? a.qk_scale * (am / (127.0f * 254.0f)) : 0.f;
#pragma unroll
        for (int kk = 0; kk < T::QSTEPS; ++kk) {
          uint32_t w1[4] = {0, 0, 0, 0}, w2[4] = {0, 0, 0, 0};
          // k-slot 16g + j of int8 k-step kk <-> d as laid out in the K chunk:
          // j < 8 at 64 kk + 8 g + j, else at 64 kk + 32 + 8 g + (j - 8)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float v = qrow_ok ? (j < 8 ? xr[2 * kk][j] : xr[2 * kk + 1][j - 8]) * inv : 0.f;
            const float c1 = fmaxf(fminf(rintf(v), 127.f), -127.f);
            const float c2 = fmaxf(fminf(rintf((v - c1) * 254.0f), 127.f), -127.f);
            if constexpr (T::PACK) {  // this lane's piece only (a per-element select)
              w1[j >> 2] |= ((uint32_t)(int)(second_piece ? c2 : c1) & 0xFFu) << (8 * (j & 3));
            } else {
              w1[j >> 2] |= ((uint32_t)(int)c1 & 0xFFu) << (8 * (j & 3));
              w2[j >> 2] |= ((uint32_t)(int)c2 & 0xFFu) << (8 * (j & 3));
            }
          }
          if constexpr (T::PACK) {
            qv[kk] = make_uint4(w1[0], w1[1], w1[2], w1[3]);
          } else {
            qv[2 * kk] = make_uint4(w1[0], w1[1], w1[2], w1[3]);
            qv[2 * kk + 1] = make_uint4(w2[0], w2[1], w2[2], w2[3]);
          }
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
            const float v = qrow_ok ? ldexpf(xr[kk][e], 8 - ex) : 0.f;
            qh16[e] = (_Float16)v;
            ql16[e] = (_Float16)(v - (float)qh16[e]);
          }
          if constexpr (T::PACK) {  // this lane's piece only (a per-element select)
            f16x8 mine;
#pragma unroll
            for (int e = 0; e < 8; ++e) mine[e] = second_piece ? ql16[e] : qh16[e];
            qv[kk] = bitcast<uint4>(mine);
          } else {
            qv[2 * kk] = bitcast<uint4>(qh16);
            qv[2 * kk + 1] = bitcast<uint4>(ql16);
          }
        }
      }
      // the other first blocks, once the query no longer needs the wave
      stage_first(1, T::RING_S - 1);
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
      // the rotated rows' LDS (merge area, or the rings' last stages, which
      // the block loop refills first) is free again; ring formats read it
      // with self-waiting accesses, so a bare barrier suffices there
      if constexpr (T::QROT) {
        if constexpr (T::RING) __builtin_amdgcn_s_barrier();
        else __syncthreads();
      }
    }

    if (FUSED && late_append) {
      store_new_tokens<FMT, D>(nr, a, geo, b, h, L, mlo, mhi, lane);
      if (kmine == T::RING_S - 1) wait_vmcnt<0>();  // staged by the first iteration's refill
    }

    // ---- stream this wave's token blocks: blk0 + wave, blk0 + wave + 4, ...
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
    // Online softmax of one block's scores: rescale l and O (and the p of a
    // block held for a paired product) past the slack, then p = 2^(s - m).
    auto softmax_phase = [&](const float (&sc)[4], float (&p)[4], float (&p_held)[4]) {
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
#pragma unroll
        for (int e = 0; e < 4; ++e) p_held[e] *= corr;  // this lane's row, like l
        m_run = m_new;
      }
      // a row that has seen no visible key yet has m_run = -inf and only
      // -inf scores: subtract 0 instead so that exp2 gives 0, not NaN
      const float m_use = (m_run == NEG_INF) ? 0.f : m_run;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = fast_exp2(sc[e] - m_use);
        l_run += p[e];
      }
    };
    // O += P . V of one block (16 tokens: 16x16x16 products)
    auto pv_single = [&](Buf<FMT, D>& buf, int jb, const float (&p)[4]) {
      const int t0 = 16 * jb;
      const f16x4 P = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
      if (__builtin_expect(t0 + 16 > L, 0)) clear_tail<FMT, D>(buf, L - t0, g);  // only the last block
      // keep the compiler from hoisting every V conversion ahead of the
      // products (it would hold all of them live and spill)
#pragma unroll
      for (int nt = 0; nt < T::NT; ++nt) {
        if ((nt & 3) == 0) __builtin_amdgcn_sched_barrier(0);
        O[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(P, v_operand<FMT, D>(buf, nt, lane), O[nt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto pv_phase = [&](Buf<FMT, D>& buf, int jb, const float (&sc)[4]) {
      float p[4], none[4] = {0.f, 0.f, 0.f, 0.f};
      softmax_phase(sc, p, none);
      pv_single(buf, jb, p);
    };
    // O += P . V of two blocks at once with 16x16x32 products: k-slots
    // 8 g .. 8 g + 3 are tokens 4 g .. 4 g + 3 of the first block and
    // 8 g + 4 .. 8 g + 7 the same tokens of the second, in P (A operand) as
    // in V (B operand).  One product costs what a 16x16x16 one does.
    auto pv_pair = [&](const float (&p0)[4], Buf<FMT, D>& b0, const float (&p1)[4], Buf<FMT, D>& b1) {
      const f16x8 P = {(_Float16)p0[0], (_Float16)p0[1], (_Float16)p0[2], (_Float16)p0[3],
                       (_Float16)p1[0], (_Float16)p1[1], (_Float16)p1[2], (_Float16)p1[3]};
#pragma unroll
      for (int nt = 0; nt < T::NT; ++nt) {
        if ((nt & 3) == 0) __builtin_amdgcn_sched_barrier(0);
        const f16x4 v0 = v_operand<FMT, D>(b0, nt, lane), v1 = v_operand<FMT, D>(b1, nt, lane);
        const f16x8 V = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P, V, O[nt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    {
      const int jend = blk0 + nblk;
      int j = blk0 + wave;
      if constexpr (T::RING) {
        // this wave's blocks j_k = blk0 + wave + 4 k, k < nk; block k sits in
        // stage k % S, and blocks k + 1 .. k + S - 1 are in flight meanwhile
        // (the first S - 1 were staged before the query setup)
        constexpr int S = T::RING_S;
        Buf<FMT, D> A;
        float sc[4];
        int st = 0;
        // Two workgroups share each SIMD, and the instruction arbiter
        // favours the older wave: left alone, one wave finishes long before
        // the other, which then runs its last blocks without a partner to
        // hide its stalls.  Stepping the priority down as a wave progresses
        // lets the one behind catch up, so the two finish close together.
        // Even so the younger workgroup of a CU (dispatched once every CU
        // has one) ended about 5 us after the older one at 1 x 262K tokens
        // (per-wave clock stamps, every run alike); it steps down at 3/8,
        // 5/8 and 7/8 of its blocks instead of 1/4, 1/2 and 3/4 (for grids
        // of one resident round, whose dispatch order is known).
        const bool young = (int)blockIdx.x >= a.pace_cus && (int)blockIdx.x < a.pace_round;
        const int q1 = young ? (3 * nk) >> 3 : nk >> 2, q2 = young ? (5 * nk) >> 3 : nk >> 1,
                  q3 = young ? (7 * nk) >> 3 : nk - (nk >> 2);
        auto pace = [&](int k) {
          if (k == q1) __builtin_amdgcn_s_setprio(2);
          if (k == q2) __builtin_amdgcn_s_setprio(1);
          if (k == q3) __builtin_amdgcn_s_setprio(0);
        };
        // refill the stage block k - 1 left with block k + S - 1, wait for
        // block k; returns its stage
        auto arrive = [&](int k) -> uint32_t {
          if (k + S - 1 < nk) {
            const int sn = st == 0 ? S - 1 : st - 1;
            stage_block<FMT, D>(ring0 + sn * T::STAGE, head0, geo, bt_row, j + 4 * (S - 1), lane);
          }
          wait_staged<T::NDMA, S>(min(S - 1, nk - 1 - k));
          return ring0 + st * T::STAGE;
        };
        auto advance = [&]() {
          j += 4;
          st = st + 1 == S ? 0 : st + 1;
        };
        if constexpr (T::PV_PAIR) {
          // blocks in pairs: the first one's p and V operands wait in
          // registers (its stage is refilled meanwhile) for the second
          Buf<FMT, D> H;
          float ph[4], p[4];
          int k = 0;
          for (; k + 1 < nk; k += 2) {
            uint32_t stg = arrive(k);
            read_stage_k<FMT, D>(A, stg, lane);
            qk_phase(A, j, sc);
            read_stage_v<FMT, D>(H, stg, lane);
            float none[4] = {0.f, 0.f, 0.f, 0.f};
            softmax_phase(sc, ph, none);
            if (__builtin_expect(16 * j + 16 > L, 0)) clear_tail<FMT, D>(H, L - 16 * j, g);
            advance();
            pace(k);
            stg = arrive(k + 1);
            read_stage_k<FMT, D>(A, stg, lane);
            qk_phase(A, j, sc);
            read_stage_v<FMT, D>(A, stg, lane);
            softmax_phase(sc, p, ph);
            if (__builtin_expect(16 * j + 16 > L, 0)) clear_tail<FMT, D>(A, L - 16 * j, g);
            pv_pair(ph, H, p, A);
            advance();
            pace(k + 1);
          }
          if (k < nk) {  // an odd last block
            const uint32_t stg = arrive(k);
            read_stage_k<FMT, D>(A, stg, lane);
            qk_phase(A, j, sc);
            read_stage_v<FMT, D>(A, stg, lane);
            pv_phase(A, j, sc);
            advance();
          }
        } else {
          for (int k = 0; k < nk; ++k) {
            const uint32_t stg = arrive(k);
            read_stage_k<FMT, D>(A, stg, lane);
            qk_phase(A, j, sc);
            read_stage_v<FMT, D>(A, stg, lane);
            pv_phase(A, j, sc);
            advance();
            pace(k);
          }
        }
        // a wave with no blocks here still has its first copies in flight
        // (clamped to a valid block); they must land before the merge
        // reuses the ring's LDS
        wait_vmcnt<0>();
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

    // ---- merge the 4 waves (the workgroup waits on its barriers: above the
    //      other workgroup's streaming waves, below a starting segment)
    __builtin_amdgcn_s_setprio(2);
    l_run = sum_over_g(l_run);
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

    // ---- write: one wave per row, summing the 4 waves' rescaled parts
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
#pragma unroll
      for (int ww = 1; ww < 4; ++ww)
#pragma unroll
        for (int i = 0; i < E; ++i) xo[i] += sm_o[(ww * Rt + row) * D + E * lane + i];
      if (!direct) {
        // the partial leaves in the original domain (the rotation is linear,
        // so merging rotated-back partials equals rotating the merged one
        // back), which lets the combine split a row across workgroups
        if constexpr (T::VROT) {
          fwht_wave<E>(xo, lane);
#pragma unroll
          for (int i = 0; i < E; ++i) xo[i] *= 0.0625f;
        }
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
// A (unit, row) item's partials: those of workgroups wa .. wb, whose ranges
// cover the unit's blocks.  Units finished by the split kernel (one
// workgroup, write_direct) have nothing to merge; empty sequences get
// out = 0, lse = -inf.

struct CombineItem {
  int64_t orow;     // output row
  int64_t slot;     // the first partial's slot row, (u + wa) * R + rr
  int nseg;         // partials to merge; 0: empty sequence, -1: written by the split kernel
};

__device__ __forceinline__ CombineItem combine_item(const DecodeArgs& a, int H_kv, unsigned item) {
  CombineItem it;
  const int u = (int)(item / (unsigned)a.R), rr = (int)(item - (unsigned)u * a.R);
  const int b = u / H_kv, h = u - b * H_kv;
  const int qi = rr / a.G, qh = h * a.G + (rr - qi * a.G);
  it.orow = ((int64_t)b * a.n_q + qi) * a.H_q + qh;
  // the sequence's blocks come from the split kernel's prefix table, so the
  // three loads go out together instead of one after seq_lens[b]
  const int cb = a.ws_cum[b], cb1 = a.ws_cum[b + 1], total = a.ws_cum[a.B];
  const int nb = (cb1 - cb) / H_kv;
  if (nb == 0) {
    it.slot = 0;
    it.nseg = 0;
    return it;
  }
  const int c = a.seg_cost, units = a.B * H_kv;
  const int64_t C = total + (int64_t)c * (units > 1 ? units - 1 : 0);
  const int ways = split_ways(C, a.nwg);
  const int64_t start = cb + h * nb + (int64_t)c * u;  // cost position of the unit's block 0
  const int wa = split_range_of(C, ways, start), wb = split_range_of(C, ways, start + nb - 1);
  it.slot = (int64_t)(u + wa) * a.R + rr;
  it.nseg = wa == wb && a.write_direct ? -1 : wb - wa + 1;
  return it;
}

// Merges partials g, g + SG, ... < nseg of 4 columns into (m, l, acc) with
// a running maximum, rescaling what is held when the maximum grows (the
// same log-sum-exp merge as the split kernel's).  Up to KF partials are in
// flight per thread: their loads go out together, so a unit split many
// ways costs about one memory round trip, not one per partial.
template <int SG>
__device__ __forceinline__ void merge_partials(const float* ml, const float* po, int nseg, int g, int64_t sml,
                                               int64_t so, float& m, float& l, float4& acc) {
  constexpr float NEG_INF = -__builtin_inff();
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
  constexpr int KF = 8;
  int s = g;
  for (; s + (KF - 1) * SG < nseg; s += KF * SG) {
    float ms[KF], ls[KF];
    float4 os[KF];
#pragma unroll
    for (int i = 0; i < KF; ++i) {
      ms[i] = ml[(s + i * SG) * sml];
      ls[i] = ml[(s + i * SG) * sml + 1];
      os[i] = *reinterpret_cast<const float4*>(po + (s + i * SG) * so);
    }
#pragma unroll
    for (int i = 0; i < KF; ++i) take(ms[i], ls[i], os[i]);
  }
  float ms[KF - 1], ls[KF - 1];
  float4 os[KF - 1];
#pragma unroll
  for (int i = 0; i < KF - 1; ++i) {
    if (s + i * SG < nseg) {
      ms[i] = ml[(s + i * SG) * sml];
      ls[i] = ml[(s + i * SG) * sml + 1];
      os[i] = *reinterpret_cast<const float4*>(po + (s + i * SG) * so);
    }
  }
#pragma unroll
  for (int i = 0; i < KF - 1; ++i)
    if (s + i * SG < nseg) take(ms[i], ls[i], os[i]);
}

// One workgroup of SG x DL threads per (unit, row, column slice), DL =
// D / (4 NS) threads per slice of D / NS columns; thread (g, c) owns columns
// 4c .. 4c + 3 of the slice and merges partials g, g + SG, ...; the groups
// then merge through LDS.  The partials are already in the original domain,
// so a row's slices are independent: a unit split many ways spreads its
// partials' bytes over NS workgroups.

template <int D, int SG, int NS>
__global__ __launch_bounds__(SG * D / (4 * NS)) void decode_combine_kernel(DecodeArgs a, int H_kv) {
  constexpr float NEG_INF = -__builtin_inff();
  constexpr int DL = D / (4 * NS);  // threads per partial slice (4 columns each)
  __shared__ float4 sacc[SG][DL];
  __shared__ float sm[SG], sl[SG];
  const int tid = threadIdx.x, c = tid % DL, g = tid / DL;
  const unsigned item = blockIdx.x / (unsigned)NS;
  const int col0 = (int)(blockIdx.x - item * (unsigned)NS) * (D / NS) + 4 * c;
  const bool lse_writer = col0 == 0;  // thread 0 of slice 0
  const CombineItem it = combine_item(a, H_kv, item);
  if (it.nseg == 0) {
    if (tid < DL) *reinterpret_cast<float4*>(a.out + it.orow * D + col0) = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.lse != nullptr && lse_writer && tid == 0) a.lse[it.orow] = NEG_INF;
    return;
  }
  if (it.nseg < 0) return;
  float m = NEG_INF, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  merge_partials<SG>(a.ws_ml + it.slot * 2, a.ws_o + it.slot * D + col0, it.nseg, g, (int64_t)a.R * 2,
                     (int64_t)a.R * D, m, l, acc);

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
  *reinterpret_cast<float4*>(a.out + it.orow * D + col0) = make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
  if (a.lse != nullptr && lse_writer && tid == 0)
    a.lse[it.orow] = Lt > 0.f ? (M + __log2f(Lt)) * 0.69314718055994531f : NEG_INF;
}

// Fewer than two partials per unit on average (many units, most finished
// by the split kernel): 256 threads take 1024 / D rows, one group of D / 4
// threads per row merging its partials alone, so the launch is not one
// small workgroup per row.  The result equals decode_combine_kernel's with
// SG = NS = 1 bit for bit.

template <int D>
__global__ __launch_bounds__(256) void decode_combine_rows_kernel(DecodeArgs a, int H_kv, int64_t rows) {
  constexpr float NEG_INF = -__builtin_inff();
  constexpr int DL = D / 4, RW = 256 / DL;
  const int tid = threadIdx.x, c = tid % DL;
  const int64_t item = (int64_t)blockIdx.x * RW + tid / DL;
  if (item >= rows) return;
  const CombineItem it = combine_item(a, H_kv, (unsigned)item);
  float4* out = reinterpret_cast<float4*>(a.out + it.orow * D + 4 * c);
  if (it.nseg == 0) {
    *out = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.lse != nullptr && c == 0) a.lse[it.orow] = NEG_INF;
    return;
  }
  if (it.nseg < 0) return;
  float m = NEG_INF, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  merge_partials<1>(a.ws_ml + it.slot * 2, a.ws_o + it.slot * D + 4 * c, it.nseg, 0, (int64_t)a.R * 2,
                    (int64_t)a.R * D, m, l, acc);
  const float inv = l > 0.f ? a.v_out_scale / l : 0.f;
  *out = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (a.lse != nullptr && c == 0) a.lse[it.orow] = l > 0.f ? (m + __log2f(l)) * 0.69314718055994531f : NEG_INF;
}

// ----------------------------------------------------------- launchers


size_t decode_split_lds_bytes(const Geometry& geo, int B, int R) {
#define KVQ_LDS_CASE(F, DD) \
  if (geo.fmt == F && geo.D == DD) return split_lds_bytes<F, DD>(B, R);
  KVQ_FOR_EACH_DECODE(KVQ_LDS_CASE)
#undef KVQ_LDS_CASE
  return 0;
}

hipError_t decode_split_occupancy(const Geometry& geo, int B, int R, int* blocks_per_cu) {
  const size_t lds = decode_split_lds_bytes(geo, B, R);
  if (R <= PACK_MAX_ROWS) {
#define KVQ_OCC_PACKED(F, DD)                                                                                      \
  if (geo.fmt == F && geo.D == DD)                                                                                 \
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, decode_split_kernel<F | VARIANT_PACK, DD, false>, \
                                                        256, lds);
    KVQ_FOR_EACH_PACKED(KVQ_OCC_PACKED)
#undef KVQ_OCC_PACKED
  }
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
  if (a.q_mx) {  // the variant keeps the MXFP8 kernel's LDS layout
    if (geo.fmt != F_MXFP8) return hipErrorInvalidValue;
#define KVQ_QMX_CASE(DD)                                                                                      \
  if (geo.D == DD) {                                                                                          \
    if (a.pool_w != nullptr)                                                                                  \
      hipLaunchKernelGGL((decode_split_kernel<F_MXFP8 | VARIANT_QMX, DD, true>), dim3(a.nwg, tiles), dim3(256), lds, \
                         stream, geo, a);                                                                     \
    else                                                                                                      \
      hipLaunchKernelGGL((decode_split_kernel<F_MXFP8 | VARIANT_QMX, DD, false>), dim3(a.nwg, tiles), dim3(256), lds, \
                         stream, geo, a);                                                                     \
    return hipGetLastError();                                                                                 \
  }
    KVQ_QMX_CASE(128) KVQ_QMX_CASE(256)
#undef KVQ_QMX_CASE
    return hipErrorInvalidValue;
  }
  // at most 8 rows: the packed kernel (same LDS layout, one tile)
  if (a.R <= PACK_MAX_ROWS) {
#define KVQ_PACKED_CASE(F, DD)                                                                                \
  if (geo.fmt == F && geo.D == DD) {                                                                          \
    if (a.pool_w != nullptr)                                                                                  \
      hipLaunchKernelGGL((decode_split_kernel<F | VARIANT_PACK, DD, true>), dim3(a.nwg, 1), dim3(256), lds, stream, \
                         geo, a);                                                                             \
    else                                                                                                      \
      hipLaunchKernelGGL((decode_split_kernel<F | VARIANT_PACK, DD, false>), dim3(a.nwg, 1), dim3(256), lds, stream, \
                         geo, a);                                                                             \
    return hipGetLastError();                                                                                 \
  }
    KVQ_FOR_EACH_PACKED(KVQ_PACKED_CASE)
#undef KVQ_PACKED_CASE
  }
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
  // about the partials per unit: under 2, several rows per workgroup; up to
  // 16 merged side by side in one workgroup per row; more (a few long
  // sequences over the whole grid) in 16 or 32 groups per 64-column slice,
  // so that a row's partials are read by D / 64 workgroups
  const int64_t expect = a.nwg / units + 1;
#define KVQ_COMBINE(DD, SG, NS)                                                                        \
  hipLaunchKernelGGL((decode_combine_kernel<DD, SG, NS>), dim3((unsigned)(rows * NS)), dim3(SG * DD / (4 * NS)), 0, \
                     stream, a, geo.H_kv)
#define KVQ_COMBINE_D(DD)                                                           \
  if (expect >= 32) KVQ_COMBINE(DD, 32, DD / 64);                                   \
  else if (expect >= 16) KVQ_COMBINE(DD, 16, DD / 64);                              \
  else if (expect >= 8) KVQ_COMBINE(DD, 8, 1);                                      \
  else if (expect >= 4) KVQ_COMBINE(DD, 4, 1);                                      \
  else if (expect >= 2) KVQ_COMBINE(DD, 2, 1);                                      \
  else hipLaunchKernelGGL((decode_combine_rows_kernel<DD>), dim3((unsigned)((rows + 1024 / DD - 1) / (1024 / DD))), \
                          dim3(256), 0, stream, a, geo.H_kv, rows);
  if (geo.D == 256) { KVQ_COMBINE_D(256) }
  else if (geo.D == 128) { KVQ_COMBINE_D(128) }
  else return hipErrorInvalidValue;
#undef KVQ_COMBINE_D
#undef KVQ_COMBINE
  return hipGetLastError();
}

}  // namespace kvq
