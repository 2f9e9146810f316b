// kvq_api.hip -- the C ABI: argument validation, split planning, launches.
//
// Every argument check the host can make happens before the first HIP call,
// so a rejected call enqueues nothing (and the checks run without a GPU).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/kvq.h"
#include "kvq_format.hpp"
#include "kvq_internal.hpp"

using namespace kvq;

namespace {

kvq_status check_desc(const kvq_cache_desc* d) {
  if (d == nullptr) return KVQ_ERR_INVALID_ARGUMENT;
  if (d->format < 0 || d->format >= F_COUNT) return KVQ_ERR_INVALID_ARGUMENT;
  if (d->num_kv_heads < 1 || d->num_pages < 1 || d->head_dim < 1 || d->page_size < 1) return KVQ_ERR_INVALID_ARGUMENT;
  if (!supported(d->format, d->head_dim, d->page_size)) return KVQ_ERR_UNSUPPORTED;
  if (d->format == F_FP8_TENSOR) {
    if (!(d->k_scale > 0.0f) || !(d->v_scale > 0.0f) || !isfinite(d->k_scale) || !isfinite(d->v_scale))
      return KVQ_ERR_INVALID_ARGUMENT;
  }
  return KVQ_OK;
}

Geometry geo_of(const kvq_cache_desc* d) { return make_geometry(d->format, d->head_dim, d->page_size, d->num_kv_heads); }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int MAX_ROWS = 1024;  // G * n_q per kv head

struct Plan {
  int32_t R, tiles, units, pps, nsplit;
  size_t ml_bytes, o_bytes;
};

kvq_status check_decode_shape(const kvq_cache_desc* d, int32_t batch, int32_t n_q, int32_t H_q, int32_t max_pages) {
  kvq_status st = check_desc(d);
  if (st != KVQ_OK) return st;
  if (batch < 0 || n_q < 1 || H_q < 1 || max_pages < 1) return KVQ_ERR_INVALID_ARGUMENT;
  if (H_q % d->num_kv_heads != 0) return KVQ_ERR_INVALID_ARGUMENT;
  if ((int64_t)(H_q / d->num_kv_heads) * n_q > MAX_ROWS) return KVQ_ERR_UNSUPPORTED;
  if ((int64_t)batch * d->num_kv_heads > (1 << 24)) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

// pages_per_split = 0: choose so that the whole problem makes about eight
// workgroups per compute unit (enough to fill 256 CUs and to even out
// sequences of different lengths), never less than one page per split.
kvq_status make_plan(const kvq_cache_desc* d, int32_t batch, int32_t n_q, int32_t H_q, int32_t max_pages,
                     int32_t pps_req, Plan* p) {
  p->R = (H_q / d->num_kv_heads) * n_q;
  p->tiles = (p->R + 15) / 16;
  p->units = batch * d->num_kv_heads;
  if (pps_req < 0) return KVQ_ERR_INVALID_ARGUMENT;
  if (pps_req > 0) {
    p->pps = pps_req < max_pages ? pps_req : max_pages;
  } else {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KVQ_ERR_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      return KVQ_ERR_HIP;
    const int64_t target = (int64_t)cus * 8;
    const int64_t work = (int64_t)p->units * p->tiles * max_pages;
    int64_t pps = (work + target - 1) / target;
    if (pps < 1) pps = 1;
    if (pps > max_pages) pps = max_pages;
    p->pps = (int32_t)pps;
  }
  p->nsplit = (max_pages + p->pps - 1) / p->pps;
  if ((int64_t)p->nsplit * p->units > INT32_MAX || p->tiles > 65535) return KVQ_ERR_UNSUPPORTED;
  const size_t rows = (size_t)p->units * p->nsplit * p->R;
  p->ml_bytes = (rows * 2 * sizeof(float) + 255) / 256 * 256;
  p->o_bytes = rows * (size_t)d->head_dim * sizeof(float);
  return KVQ_OK;
}

DecodeArgs base_args(const kvq_cache_desc* d, const Plan& p, int32_t batch, int32_t n_q, int32_t H_q,
                     int32_t max_pages, const int32_t* seq_lens, float softmax_scale) {
  DecodeArgs a{};
  a.seq_lens = seq_lens;
  a.B = batch; a.n_q = n_q; a.H_q = H_q; a.G = H_q / d->num_kv_heads; a.R = p.R;
  a.max_pages = max_pages; a.pps = p.pps; a.nsplit = p.nsplit;
  a.qk_scale = softmax_scale * 1.4426950408889634f * (d->format == F_FP8_TENSOR ? d->k_scale : 1.0f);
  a.v_out_scale = d->format == F_FP8_TENSOR ? d->v_scale : 1.0f;
  return a;
}

kvq_status hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

}  // namespace

extern "C" {

const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARGUMENT: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported format / head_dim / page_size / shape";
    case KVQ_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KVQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

kvq_status kvq_page_bytes(const kvq_cache_desc* desc, size_t* bytes_per_page) {
  kvq_status st = check_desc(desc);
  if (st != KVQ_OK) return st;
  if (bytes_per_page == nullptr) return KVQ_ERR_INVALID_ARGUMENT;
  *bytes_per_page = (size_t)geo_of(desc).page_bytes;
  return KVQ_OK;
}

kvq_status kvq_quantize_append(const kvq_cache_desc* desc, void* pool, const void* k_bf16, const void* v_bf16,
                               int64_t num_tokens, const int32_t* slot_mapping, hipStream_t stream) {
  kvq_status st = check_desc(desc);
  if (st != KVQ_OK) return st;
  if (num_tokens < 0) return KVQ_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return KVQ_OK;
  if (pool == nullptr || k_bf16 == nullptr || v_bf16 == nullptr || slot_mapping == nullptr)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (!aligned(pool, 128) || !aligned(k_bf16, 16) || !aligned(v_bf16, 16)) return KVQ_ERR_INVALID_ARGUMENT;
  if (num_tokens * desc->num_kv_heads > ((int64_t)1 << 40)) return KVQ_ERR_UNSUPPORTED;
  const Geometry geo = geo_of(desc);
  return hip_status(launch_append(static_cast<uint8_t*>(pool), static_cast<const uint16_t*>(k_bf16),
                                  static_cast<const uint16_t*>(v_bf16), num_tokens, slot_mapping, geo,
                                  desc->k_scale, desc->v_scale, stream));
}

kvq_status kvq_decode_plan(const kvq_cache_desc* desc, int32_t batch, int32_t n_q, int32_t num_q_heads,
                           int32_t max_pages_per_seq, int32_t* pages_per_split, int32_t* num_splits) {
  kvq_status st = check_decode_shape(desc, batch, n_q, num_q_heads, max_pages_per_seq);
  if (st != KVQ_OK) return st;
  if (pages_per_split == nullptr || num_splits == nullptr) return KVQ_ERR_INVALID_ARGUMENT;
  Plan p;
  st = make_plan(desc, batch, n_q, num_q_heads, max_pages_per_seq, 0, &p);
  if (st != KVQ_OK) return st;
  *pages_per_split = p.pps;
  *num_splits = p.nsplit;
  return KVQ_OK;
}

kvq_status kvq_decode_workspace_size(const kvq_cache_desc* desc, int32_t batch, int32_t n_q, int32_t num_q_heads,
                                     int32_t max_pages_per_seq, int32_t pages_per_split, size_t* bytes) {
  kvq_status st = check_decode_shape(desc, batch, n_q, num_q_heads, max_pages_per_seq);
  if (st != KVQ_OK) return st;
  if (bytes == nullptr) return KVQ_ERR_INVALID_ARGUMENT;
  Plan p;
  st = make_plan(desc, batch, n_q, num_q_heads, max_pages_per_seq, pages_per_split, &p);
  if (st != KVQ_OK) return st;
  *bytes = p.ml_bytes + p.o_bytes;
  return KVQ_OK;
}

static kvq_status decode_common(const kvq_cache_desc* desc, const void* pool, const void* q_bf16, int32_t batch,
                                int32_t n_q, int32_t H_q, const int32_t* block_table, int32_t max_pages,
                                const int32_t* seq_lens, float softmax_scale, int32_t pps_req, bool allow_direct,
                                float* out, float* lse, void* workspace, size_t workspace_bytes,
                                hipStream_t stream, bool run_combine) {
  kvq_status st = check_decode_shape(desc, batch, n_q, H_q, max_pages);
  if (st != KVQ_OK) return st;
  if (!isfinite(softmax_scale)) return KVQ_ERR_INVALID_ARGUMENT;
  if (pps_req < 0) return KVQ_ERR_INVALID_ARGUMENT;
  if (batch == 0) return KVQ_OK;
  if (pool == nullptr || q_bf16 == nullptr || block_table == nullptr || seq_lens == nullptr)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (run_combine && out == nullptr) return KVQ_ERR_INVALID_ARGUMENT;
  if (!aligned(pool, 128) || !aligned(q_bf16, 16) || (out != nullptr && !aligned(out, 16)))
    return KVQ_ERR_INVALID_ARGUMENT;
  Plan p;
  st = make_plan(desc, batch, n_q, H_q, max_pages, pps_req, &p);
  if (st != KVQ_OK) return st;
  const bool direct = allow_direct && p.nsplit == 1;
  if (!direct) {
    if (workspace == nullptr || !aligned(workspace, 256)) return KVQ_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < p.ml_bytes + p.o_bytes) return KVQ_ERR_WORKSPACE_TOO_SMALL;
  }
  const Geometry geo = geo_of(desc);
  DecodeArgs a = base_args(desc, p, batch, n_q, H_q, max_pages, seq_lens, softmax_scale);
  a.pool = static_cast<const uint8_t*>(pool);
  a.q = static_cast<const uint16_t*>(q_bf16);
  a.block_table = block_table;
  a.direct = direct ? 1 : 0;
  a.out = out;
  a.lse = lse;
  if (!direct) {
    a.ws_ml = static_cast<float*>(workspace);
    a.ws_o = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + p.ml_bytes);
  }
  hipError_t e = launch_decode_split(geo, a, stream);
  if (e != hipSuccess) return KVQ_ERR_HIP;
  if (!direct && run_combine) e = launch_decode_combine(geo, a, stream);
  return hip_status(e);
}

kvq_status kvq_decode_attention(const kvq_cache_desc* desc, const void* pool, const void* q_bf16, int32_t batch,
                                int32_t n_q, int32_t num_q_heads, const int32_t* block_table,
                                int32_t max_pages_per_seq, const int32_t* seq_lens, float softmax_scale, float* out,
                                float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_common(desc, pool, q_bf16, batch, n_q, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                       softmax_scale, 0, true, out, lse, workspace, workspace_bytes, stream, true);
}

kvq_status kvq_decode_split(const kvq_cache_desc* desc, const void* pool, const void* q_bf16, int32_t batch,
                            int32_t n_q, int32_t num_q_heads, const int32_t* block_table,
                            int32_t max_pages_per_seq, const int32_t* seq_lens, float softmax_scale,
                            int32_t pages_per_split, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_common(desc, pool, q_bf16, batch, n_q, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                       softmax_scale, pages_per_split, false, nullptr, nullptr, workspace, workspace_bytes, stream,
                       false);
}

kvq_status kvq_decode_combine(const kvq_cache_desc* desc, int32_t batch, int32_t n_q, int32_t num_q_heads,
                              int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t pages_per_split,
                              const void* workspace, size_t workspace_bytes, float* out, float* lse,
                              hipStream_t stream) {
  kvq_status st = check_decode_shape(desc, batch, n_q, num_q_heads, max_pages_per_seq);
  if (st != KVQ_OK) return st;
  if (pages_per_split < 0) return KVQ_ERR_INVALID_ARGUMENT;
  if (batch == 0) return KVQ_OK;
  if (seq_lens == nullptr || out == nullptr || workspace == nullptr) return KVQ_ERR_INVALID_ARGUMENT;
  if (!aligned(out, 16) || !aligned(workspace, 256)) return KVQ_ERR_INVALID_ARGUMENT;
  Plan p;
  st = make_plan(desc, batch, n_q, num_q_heads, max_pages_per_seq, pages_per_split, &p);
  if (st != KVQ_OK) return st;
  if (workspace_bytes < p.ml_bytes + p.o_bytes) return KVQ_ERR_WORKSPACE_TOO_SMALL;
  const Geometry geo = geo_of(desc);
  DecodeArgs a = base_args(desc, p, batch, n_q, num_q_heads, max_pages_per_seq, seq_lens, 1.0f);
  a.ws_ml = const_cast<float*>(static_cast<const float*>(workspace));
  a.ws_o = reinterpret_cast<float*>(const_cast<uint8_t*>(static_cast<const uint8_t*>(workspace)) + p.ml_bytes);
  a.out = out;
  a.lse = lse;
  return hip_status(launch_decode_combine(geo, a, stream));
}

kvq_status kvq_dequant_page(const kvq_cache_desc* desc, const void* pool, int64_t page, int32_t flags, float* k_out,
                            float* v_out, hipStream_t stream) {
  kvq_status st = check_desc(desc);
  if (st != KVQ_OK) return st;
  if (pool == nullptr || k_out == nullptr || v_out == nullptr) return KVQ_ERR_INVALID_ARGUMENT;
  if (page < 0 || page >= desc->num_pages) return KVQ_ERR_INVALID_ARGUMENT;
  if ((flags & ~KVQ_DEQUANT_STORED_DOMAIN) != 0) return KVQ_ERR_INVALID_ARGUMENT;
  if (!aligned(pool, 128) || !aligned(k_out, 16) || !aligned(v_out, 16)) return KVQ_ERR_INVALID_ARGUMENT;
  const Geometry geo = geo_of(desc);
  return hip_status(launch_dequant_page(geo, static_cast<const uint8_t*>(pool), page,
                                        (flags & KVQ_DEQUANT_STORED_DOMAIN) != 0, desc->k_scale, desc->v_scale,
                                        k_out, v_out, stream));
}

}  // extern "C"
