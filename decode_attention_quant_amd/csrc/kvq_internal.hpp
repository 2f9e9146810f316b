// kvq_internal.hpp -- launchers shared between the kernel files and the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_format.hpp"

namespace kvq {

// Arguments of one decode launch.
//
// Work is scheduled stream-K style: the token blocks (16 tokens) of every
// (sequence b, kv head h) unit, units in order u = b * H_kv + h, form one
// flat range of T blocks; workgroup w of the split kernel takes a
// contiguous run of it, an equal share of a cost that adds seg_cost blocks
// between one unit and the next (split_ways and blocks_before_cost in the
// split kernel's source give the exact ranges).  A unit wholly inside one
// workgroup's range can be finished there; a unit spread over workgroups
// w_a..w_b leaves one partial (m, l, o) per workgroup, in slot u + w (the
// pairs (u, w) visited form a monotone staircase, so u + w is unique), and
// the combine kernel merges them.
struct DecodeArgs {
  const uint8_t* pool;
  const uint16_t* q;          // [B][n_q][H_q][D] bf16
  const int32_t* block_table; // [B][max_pages]
  const int32_t* seq_lens;    // [B]
  int32_t B, n_q, H_q, G, R;  // G = H_q / H_kv, R = G * n_q rows per kv head
  int32_t max_pages;
  int32_t nwg;                // workgroups of the split kernel
  int32_t seg_cost;           // blocks each unit adds to the cost the split ranges share equally
  float qk_scale;             // softmax_scale * log2(e) (* k_scale for FP8_TENSOR)
  float v_out_scale;          // v_scale for FP8_TENSOR, else 1
  int32_t* ws_cum;            // [B + 1]: H_kv * (blocks of sequences 0..b-1), written by workgroup 0
  float* ws_ml;               // [slots][R][2]: m (base 2), l
  float* ws_o;                // [slots][R][D]: unnormalized o
  float* out;                 // [B][n_q][H_q][D]
  float* lse;                 // [B][n_q][H_q], nullable
  int32_t write_direct;       // 1: finish units held by one workgroup in the split kernel
  // Dispatch order of a split grid of one resident round: of its
  // pace_round workgroups the first pace_cus take one CU each and the rest
  // join them as the younger workgroup of their CU (0: pace every workgroup
  // alike).
  int32_t pace_cus, pace_round;
  int32_t q_mx;               // 1: MXFP8 cache read with q rounded to MXFP8 (block-scaled fp8 Q.K)
  // Fused decode step (pool_w non-null): before reading a block, the split
  // workgroup that owns it encodes and stores the new tokens in it, the n_q
  // newest positions L_b - n_q .. L_b - 1 of each sequence, whose slots come
  // from the block table.  Needs R <= 16 (one row tile per block).
  uint8_t* pool_w;            // the pool, written (the same memory as pool)
  const uint16_t* k_new;      // [B][n_q][H_kv][D] bf16
  const uint16_t* v_new;      // [B][n_q][H_kv][D] bf16
  float enc_k_scale, enc_v_scale;  // per-tensor encoding scales (FP8_TENSOR)
};

// LDS bytes of the split kernel for a batch of B sequences and R rows.
size_t decode_split_lds_bytes(const Geometry& geo, int B, int R);
// Workgroups of the split kernel that fit on one CU at once.
hipError_t decode_split_occupancy(const Geometry& geo, int B, int R, int* blocks_per_cu);

hipError_t launch_append(uint8_t* pool, const uint16_t* k, const uint16_t* v, int64_t T, const int32_t* slots,
                         const Geometry& geo, float k_scale, float v_scale, hipStream_t stream);
hipError_t launch_decode_split(const Geometry& geo, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_combine(const Geometry& geo, const DecodeArgs& a, hipStream_t stream);
// Chunked-prefill attention (no split: DecodeArgs' workspace fields unused).
hipError_t launch_prefill(const Geometry& geo, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_dequant_page(const Geometry& geo, const uint8_t* pool, int64_t page, bool stored_domain,
                               float k_scale, float v_scale, float* k_out, float* v_out, hipStream_t stream);

}  // namespace kvq
