// kvq_api.hip -- the C ABI: argument validation, split planning, launches.
//
// Every argument check the host can make happens before the first HIP call,
// so a rejected call enqueues nothing (and the checks run without a GPU).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

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
  if (k_tensor_scaled(d->format) && (!(d->k_scale > 0.0f) || !isfinite(d->k_scale))) return KVQ_ERR_INVALID_ARGUMENT;
  if (v_tensor_scaled(d->format) && (!(d->v_scale > 0.0f) || !isfinite(d->v_scale))) return KVQ_ERR_INVALID_ARGUMENT;
  return KVQ_OK;
}

Geometry geo_of(const kvq_cache_desc* d) { return make_geometry(d->format, d->head_dim, d->page_size, d->num_kv_heads); }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int MAX_ROWS = 1024;   // G * n_q per kv head
constexpr int MAX_BATCH = 4096;  // the split kernel keeps a per-sequence prefix table in LDS

struct Plan {
  int32_t R, tiles, units, nwg, slots;
  int32_t cus, per_cu;  // the device's CUs and the split workgroups one holds (0: unknown)
  size_t cum_bytes, ml_bytes, o_bytes;
  size_t total() const { return cum_bytes + ml_bytes + o_bytes; }
};

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// What a split workgroup's visit to a further unit costs, in 16-token
// blocks: the query set-up, the ring's refill and the merge again (measured
// by clock stamps: 5 us more for workgroups of two units on 32 sequences of
// 8K-32K tokens, 7-12 us on 64 of 1K-128K in K8V4).  With 24 such blocks
// between units those splits ran 1.3-1.7% faster; ranges that line up with
// the units (one 262K sequence) stay as they were.
constexpr int32_t SEG_COST = 24;

kvq_status check_decode_shape(const kvq_cache_desc* d, int32_t batch, int32_t n_q, int32_t H_q, int32_t max_pages) {
  kvq_status st = check_desc(d);
  if (st != KVQ_OK) return st;
  if (batch < 0 || n_q < 1 || H_q < 1 || max_pages < 1) return KVQ_ERR_INVALID_ARGUMENT;
  if (H_q % d->num_kv_heads != 0) return KVQ_ERR_INVALID_ARGUMENT;
  if ((int64_t)(H_q / d->num_kv_heads) * n_q > MAX_ROWS) return KVQ_ERR_UNSUPPORTED;
  if (batch > MAX_BATCH) return KVQ_ERR_UNSUPPORTED;
  if ((int64_t)max_pages * d->page_size >= ((int64_t)1 << 31) / 16) return KVQ_ERR_UNSUPPORTED;
  // the flat block range and the combine grid stay within int32
  const int64_t units = (int64_t)batch * d->num_kv_heads;
  if (units * ((int64_t)max_pages * d->page_size / 16 + SEG_COST) > INT32_MAX) return KVQ_ERR_UNSUPPORTED;
  if (units * (H_q / d->num_kv_heads) * n_q > INT32_MAX) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

// num_workgroups = 0: one round of the workgroups the device holds at
// once; a positive value forces that count.  Short problems leave some of
// them empty (the kernel keeps ranges of at least 4-128 blocks).
kvq_status make_plan(const kvq_cache_desc* d, int32_t batch, int32_t n_q, int32_t H_q, int32_t max_pages,
                     int32_t nwg_req, Plan* p) {
  p->R = (H_q / d->num_kv_heads) * n_q;
  p->tiles = (p->R + 15) / 16;
  p->units = batch * d->num_kv_heads;
  if (nwg_req < 0) return KVQ_ERR_INVALID_ARGUMENT;
  p->cus = p->per_cu = 0;
  if (nwg_req > 0) {
    p->nwg = nwg_req;
    int dev = 0, cus = 0, per_cu = 0;
    const Geometry geo = make_geometry(d->format, d->head_dim, d->page_size, d->num_kv_heads);
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        decode_split_occupancy(geo, batch, p->R, &per_cu) == hipSuccess && cus > 0 && per_cu > 0) {
      p->cus = cus;
      p->per_cu = per_cu;
    }
  } else {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KVQ_ERR_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      return KVQ_ERR_HIP;
    const Geometry geo = make_geometry(d->format, d->head_dim, d->page_size, d->num_kv_heads);
    if (decode_split_occupancy(geo, batch, p->R, &per_cu) != hipSuccess || per_cu < 1) return KVQ_ERR_HIP;
    p->cus = cus;
    p->per_cu = per_cu;
    // One round of resident workgroups.  A partial last round would run a
    // few workgroups alone at the end (measured: a 640-workgroup grid on
    // 512 slots spent a third of its time on the last 128), and every
    // further round pays each workgroup's start-up and merge again
    // (measured: two rounds for 32 sequences of 8K-32K tokens were 4-6%
    // slower than one, 1.3% for 64 of 1K-128K; one workgroup per unit for
    // 8192 units of 256 blocks, 16 rounds, 1.2% slower than one round).
    p->nwg = (int32_t)((int64_t)cus * per_cu);
  }
  if (p->nwg > (1 << 24) || p->tiles > 65535) return KVQ_ERR_UNSUPPORTED;
  p->slots = p->units + p->nwg;
  p->cum_bytes = align256((size_t)(batch + 1) * sizeof(int32_t));
  p->ml_bytes = align256((size_t)p->slots * p->R * 2 * sizeof(float));
  p->o_bytes = (size_t)p->slots * p->R * (size_t)d->head_dim * sizeof(float);
  return KVQ_OK;
}

DecodeArgs base_args(const kvq_cache_desc* d, const Plan& p, int32_t batch, int32_t n_q, int32_t H_q,
                     int32_t max_pages, const int32_t* seq_lens, float softmax_scale, void* workspace) {
  DecodeArgs a{};
  a.seq_lens = seq_lens;
  a.B = batch; a.n_q = n_q; a.H_q = H_q; a.G = H_q / d->num_kv_heads; a.R = p.R;
  a.max_pages = max_pages; a.nwg = p.nwg;
  a.seg_cost = SEG_COST;
  // a grid of one resident round whose units span at least 4 workgroups
  // each on average: with more rounds the two workgroups of a CU are best
  // left staggered (pacing the first round's younger ones measured 1.5-2%
  // slower for 16 rounds), and where a workgroup holds several units
  // (64 sequences of 1K-128K tokens) the bias measured 0.9% slower
  const bool one_round = p.per_cu >= 2 && (int64_t)p.nwg <= (int64_t)p.cus * p.per_cu &&
                         (int64_t)p.units * 4 <= (int64_t)p.nwg;
  a.pace_cus = one_round ? p.cus : 0;
  a.pace_round = one_round ? p.cus * p.per_cu : 0;
  a.qk_scale = softmax_scale * 1.4426950408889634f * (k_tensor_scaled(d->format) ? d->k_scale : 1.0f);
  a.v_out_scale = v_tensor_scaled(d->format) ? d->v_scale : 1.0f;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.ws_cum = reinterpret_cast<int32_t*>(ws);
  a.ws_ml = reinterpret_cast<float*>(ws + p.cum_bytes);
  a.ws_o = reinterpret_cast<float*>(ws + p.cum_bytes + p.ml_bytes);
  return a;
}

kvq_status hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

}  // namespace

// The workspace of kvq_decode_attention_noalloc: a file-scope device array
// that every GPU the library runs on holds until the process ends.  In host
// code its name is a host-side stand-in, not a device address; kernels get
// the address hipGetSymbolAddress gives for the current device, resolved
// once per device and kept below.
static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mutex;
void* scratch_ptr[MAX_DEVICES] = {};

// The current device's address of `scratch` (nullptr on a HIP error).
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

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
                           int32_t max_pages_per_seq, int32_t* num_workgroups, int32_t* num_slots) {
  kvq_status st = check_decode_shape(desc, batch, n_q, num_q_heads, max_pages_per_seq);
  if (st != KVQ_OK) return st;
  if (num_workgroups == nullptr || num_slots == nullptr) return KVQ_ERR_INVALID_ARGUMENT;
  Plan p;
  st = make_plan(desc, batch, n_q, num_q_heads, max_pages_per_seq, 0, &p);
  if (st != KVQ_OK) return st;
  *num_workgroups = p.nwg;
  *num_slots = p.slots;
  return KVQ_OK;
}

kvq_status kvq_decode_workspace_size_for(const kvq_cache_desc* desc, int32_t batch, int32_t n_q,
                                         int32_t num_q_heads, int32_t max_pages_per_seq, int32_t num_workgroups,
                                         size_t* bytes) {
  kvq_status st = check_decode_shape(desc, batch, n_q, num_q_heads, max_pages_per_seq);
  if (st != KVQ_OK) return st;
  if (bytes == nullptr) return KVQ_ERR_INVALID_ARGUMENT;
  Plan p;
  st = make_plan(desc, batch, n_q, num_q_heads, max_pages_per_seq, num_workgroups, &p);
  if (st != KVQ_OK) return st;
  *bytes = p.total();
  return KVQ_OK;
}

kvq_status kvq_decode_workspace_size(const kvq_cache_desc* desc, int32_t batch, int32_t n_q, int32_t num_q_heads,
                                     int32_t max_pages_per_seq, size_t* bytes) {
  return kvq_decode_workspace_size_for(desc, batch, n_q, num_q_heads, max_pages_per_seq, 0, bytes);
}

static kvq_status decode_run(const kvq_cache_desc* desc, const void* pool, const void* q_bf16, int32_t batch,
                             int32_t n_q, int32_t H_q, const int32_t* block_table, int32_t max_pages,
                             const int32_t* seq_lens, float softmax_scale, int32_t nwg_req, bool write_direct,
                             bool run_split, bool run_combine, float* out, float* lse, void* workspace,
                             size_t workspace_bytes, hipStream_t stream, const void* k_new = nullptr,
                             const void* v_new = nullptr, bool q_mx = false) {
  kvq_status st = check_decode_shape(desc, batch, n_q, H_q, max_pages);
  if (st != KVQ_OK) return st;
  if (q_mx && desc->format != KVQ_MXFP8) return KVQ_ERR_UNSUPPORTED;
  if (!isfinite(softmax_scale)) return KVQ_ERR_INVALID_ARGUMENT;
  if (nwg_req < 0) return KVQ_ERR_INVALID_ARGUMENT;
  if (batch == 0) return KVQ_OK;
  if (seq_lens == nullptr || workspace == nullptr || !aligned(workspace, 256)) return KVQ_ERR_INVALID_ARGUMENT;
  if (run_split) {
    if (pool == nullptr || q_bf16 == nullptr || block_table == nullptr) return KVQ_ERR_INVALID_ARGUMENT;
    if (!aligned(pool, 128) || !aligned(q_bf16, 16)) return KVQ_ERR_INVALID_ARGUMENT;
  }
  if (write_direct || run_combine) {
    if (out == nullptr || !aligned(out, 16)) return KVQ_ERR_INVALID_ARGUMENT;
  }
  Plan p;
  st = make_plan(desc, batch, n_q, H_q, max_pages, nwg_req, &p);
  if (st != KVQ_OK) return st;
  if (workspace_bytes < p.total()) return KVQ_ERR_WORKSPACE_TOO_SMALL;
  const Geometry geo = geo_of(desc);
  DecodeArgs a = base_args(desc, p, batch, n_q, H_q, max_pages, seq_lens, softmax_scale, workspace);
  a.pool = static_cast<const uint8_t*>(pool);
  a.q = static_cast<const uint16_t*>(q_bf16);
  a.block_table = block_table;
  a.write_direct = write_direct ? 1 : 0;
  a.q_mx = q_mx ? 1 : 0;
  a.out = out;
  a.lse = lse;
  if (k_new != nullptr) {  // fused step
    a.pool_w = static_cast<uint8_t*>(const_cast<void*>(pool));
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.enc_k_scale = desc->k_scale;
    a.enc_v_scale = desc->v_scale;
  }
  hipError_t e = hipSuccess;
  if (run_split) e = launch_decode_split(geo, a, stream);
  if (e != hipSuccess) return KVQ_ERR_HIP;
  if (run_combine) e = launch_decode_combine(geo, a, stream);
  return hip_status(e);
}

kvq_status kvq_decode_attention(const kvq_cache_desc* desc, const void* pool, const void* q_bf16, int32_t batch,
                                int32_t n_q, int32_t num_q_heads, const int32_t* block_table,
                                int32_t max_pages_per_seq, const int32_t* seq_lens, float softmax_scale, float* out,
                                float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_run(desc, pool, q_bf16, batch, n_q, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                    softmax_scale, 0, true, true, true, out, lse, workspace, workspace_bytes, stream);
}

kvq_status kvq_decode_attention_noalloc(const kvq_cache_desc* desc, const void* pool, const void* q_bf16,
                                        int32_t batch, int32_t n_q, int32_t num_q_heads, const int32_t* block_table,
                                        int32_t max_pages_per_seq, const int32_t* seq_lens, float softmax_scale,
                                        float* out, float* lse, hipStream_t stream) {
  kvq_status st = check_decode_shape(desc, batch, n_q, num_q_heads, max_pages_per_seq);
  if (st != KVQ_OK) return st;
  if (batch == 0) return KVQ_OK;
  Plan p;
  st = make_plan(desc, batch, n_q, num_q_heads, max_pages_per_seq, 0, &p);
  if (st != KVQ_OK) return st;
  if (p.total() > (size_t)KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE_TOO_SMALL;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return KVQ_ERR_HIP;
  return decode_run(desc, pool, q_bf16, batch, n_q, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                    softmax_scale, 0, true, true, true, out, lse, ws, (size_t)KVQ_NOALLOC_SCRATCH_BYTES, stream);
}

kvq_status kvq_decode_step(const kvq_cache_desc* desc, void* pool, const void* k_new_bf16, const void* v_new_bf16,
                           const void* q_bf16, int32_t batch, int32_t n_q, int32_t num_q_heads,
                           const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                           float softmax_scale, float* out, float* lse, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  kvq_status st = check_decode_shape(desc, batch, n_q, num_q_heads, max_pages_per_seq);
  if (st != KVQ_OK) return st;
  // one row tile: the workgroup that owns a block is its only reader
  if ((num_q_heads / desc->num_kv_heads) * n_q > 16) return KVQ_ERR_UNSUPPORTED;
  if (batch > 0) {
    if (k_new_bf16 == nullptr || v_new_bf16 == nullptr) return KVQ_ERR_INVALID_ARGUMENT;
    if (!aligned(k_new_bf16, 16) || !aligned(v_new_bf16, 16)) return KVQ_ERR_INVALID_ARGUMENT;
  }
  return decode_run(desc, pool, q_bf16, batch, n_q, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                    softmax_scale, 0, true, true, true, out, lse, workspace, workspace_bytes, stream, k_new_bf16,
                    v_new_bf16);
}

kvq_status kvq_decode_step_split(const kvq_cache_desc* desc, void* pool, const void* k_new_bf16,
                                 const void* v_new_bf16, const void* q_bf16, int32_t batch, int32_t n_q,
                                 int32_t num_q_heads, const int32_t* block_table, int32_t max_pages_per_seq,
                                 const int32_t* seq_lens, float softmax_scale, int32_t num_workgroups,
                                 int32_t flags, float* out, float* lse, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if ((flags & ~(KVQ_SPLIT_WRITE_WHOLE_UNITS | KVQ_SPLIT_Q_MXFP8)) != 0) return KVQ_ERR_INVALID_ARGUMENT;
  kvq_status st = check_decode_shape(desc, batch, n_q, num_q_heads, max_pages_per_seq);
  if (st != KVQ_OK) return st;
  if ((num_q_heads / desc->num_kv_heads) * n_q > 16) return KVQ_ERR_UNSUPPORTED;
  if (batch > 0) {
    if (k_new_bf16 == nullptr || v_new_bf16 == nullptr) return KVQ_ERR_INVALID_ARGUMENT;
    if (!aligned(k_new_bf16, 16) || !aligned(v_new_bf16, 16)) return KVQ_ERR_INVALID_ARGUMENT;
  }
  const bool whole = (flags & KVQ_SPLIT_WRITE_WHOLE_UNITS) != 0;
  return decode_run(desc, pool, q_bf16, batch, n_q, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                    softmax_scale, num_workgroups, whole, true, false, whole ? out : nullptr, whole ? lse : nullptr,
                    workspace, workspace_bytes, stream, k_new_bf16, v_new_bf16, (flags & KVQ_SPLIT_Q_MXFP8) != 0);
}

kvq_status kvq_decode_split(const kvq_cache_desc* desc, const void* pool, const void* q_bf16, int32_t batch,
                            int32_t n_q, int32_t num_q_heads, const int32_t* block_table,
                            int32_t max_pages_per_seq, const int32_t* seq_lens, float softmax_scale,
                            int32_t num_workgroups, int32_t flags, float* out, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if ((flags & ~(KVQ_SPLIT_WRITE_WHOLE_UNITS | KVQ_SPLIT_Q_MXFP8)) != 0) return KVQ_ERR_INVALID_ARGUMENT;
  const bool whole = (flags & KVQ_SPLIT_WRITE_WHOLE_UNITS) != 0;
  return decode_run(desc, pool, q_bf16, batch, n_q, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                    softmax_scale, num_workgroups, whole, true, false, whole ? out : nullptr,
                    whole ? lse : nullptr, workspace, workspace_bytes, stream, nullptr, nullptr,
                    (flags & KVQ_SPLIT_Q_MXFP8) != 0);
}

kvq_status kvq_decode_combine(const kvq_cache_desc* desc, int32_t batch, int32_t n_q, int32_t num_q_heads,
                              int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t num_workgroups,
                              int32_t flags, const void* workspace, size_t workspace_bytes, float* out, float* lse,
                              hipStream_t stream) {
  // KVQ_SPLIT_Q_MXFP8 changes only the split phase: accepted and ignored here
  if ((flags & ~(KVQ_SPLIT_WRITE_WHOLE_UNITS | KVQ_SPLIT_Q_MXFP8)) != 0) return KVQ_ERR_INVALID_ARGUMENT;
  return decode_run(desc, nullptr, nullptr, batch, n_q, num_q_heads, nullptr, max_pages_per_seq, seq_lens, 1.0f,
                    num_workgroups, (flags & KVQ_SPLIT_WRITE_WHOLE_UNITS) != 0, false, true, out, lse,
                    const_cast<void*>(workspace), workspace_bytes, stream);
}

kvq_status kvq_prefill_attention(const kvq_cache_desc* desc, const void* pool, const void* q_bf16, int32_t batch,
                                 int32_t n_q, int32_t num_q_heads, const int32_t* block_table,
                                 int32_t max_pages_per_seq, const int32_t* seq_lens, float softmax_scale, float* out,
                                 float* lse, hipStream_t stream) {
  kvq_status st = check_desc(desc);
  if (st != KVQ_OK) return st;
  if (batch < 0 || n_q < 1 || num_q_heads < 1 || max_pages_per_seq < 1) return KVQ_ERR_INVALID_ARGUMENT;
  if (num_q_heads % desc->num_kv_heads != 0) return KVQ_ERR_INVALID_ARGUMENT;
  if (!isfinite(softmax_scale)) return KVQ_ERR_INVALID_ARGUMENT;
  const int64_t G = num_q_heads / desc->num_kv_heads;
  const int64_t R = G * n_q;
  const int64_t work = (int64_t)batch * desc->num_kv_heads * ((R + 63) / 64);
  if (R > INT32_MAX / 2 || work > (int64_t)1 << 30) return KVQ_ERR_UNSUPPORTED;
  if ((int64_t)max_pages_per_seq * desc->page_size >= ((int64_t)1 << 31) / 16) return KVQ_ERR_UNSUPPORTED;
  if (batch == 0) return KVQ_OK;
  if (pool == nullptr || q_bf16 == nullptr || block_table == nullptr || seq_lens == nullptr || out == nullptr)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (!aligned(pool, 128) || !aligned(q_bf16, 16) || !aligned(out, 16)) return KVQ_ERR_INVALID_ARGUMENT;
  DecodeArgs a{};
  a.pool = static_cast<const uint8_t*>(pool);
  a.q = static_cast<const uint16_t*>(q_bf16);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.B = batch; a.n_q = n_q; a.H_q = num_q_heads; a.G = (int32_t)G; a.R = (int32_t)R;
  a.max_pages = max_pages_per_seq;
  a.qk_scale = softmax_scale * 1.4426950408889634f * (k_tensor_scaled(desc->format) ? desc->k_scale : 1.0f);
  a.v_out_scale = v_tensor_scaled(desc->format) ? desc->v_scale : 1.0f;
  a.out = out;
  a.lse = lse;
  return hip_status(launch_prefill(geo_of(desc), a, stream));
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
