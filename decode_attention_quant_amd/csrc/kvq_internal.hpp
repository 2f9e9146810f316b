// kvq_internal.hpp -- launchers shared between the kernel files and the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_format.hpp"

namespace kvq {

// Arguments of one decode launch (split or direct mode).
struct DecodeArgs {
  const uint8_t* pool;
  const uint16_t* q;          // [B][n_q][H_q][D] bf16
  const int32_t* block_table; // [B][max_pages]
  const int32_t* seq_lens;    // [B]
  int32_t B, n_q, H_q, G, R;  // G = H_q / H_kv, R = G * n_q rows per kv head
  int32_t max_pages, pps, nsplit;
  float qk_scale;             // softmax_scale * log2(e) (* k_scale for FP8_TENSOR)
  float v_out_scale;          // v_scale for FP8_TENSOR, else 1
  float* ws_ml;               // split mode: [units][nsplit][R][2]
  float* ws_o;                // split mode: [units][nsplit][R][D]
  float* out;                 // direct mode: [B][n_q][H_q][D]
  float* lse;                 // direct mode, nullable
  int32_t direct;             // 1: one split per sequence, write out/lse directly
};

hipError_t launch_append(uint8_t* pool, const uint16_t* k, const uint16_t* v, int64_t T, const int32_t* slots,
                         const Geometry& geo, float k_scale, float v_scale, hipStream_t stream);
hipError_t launch_decode_split(const Geometry& geo, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_combine(const Geometry& geo, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_dequant_page(const Geometry& geo, const uint8_t* pool, int64_t page, bool stored_domain,
                               float k_scale, float v_scale, float* k_out, float* v_out, hipStream_t stream);

}  // namespace kvq
