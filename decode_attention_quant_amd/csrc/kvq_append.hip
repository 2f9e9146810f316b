// kvq_append.hip -- quantize-append: encode bf16 K/V rows and store them in
// the paged pool (the write path of every format of the NInfer KV-cache
// quantization guide, section on the five formats; TokenSpeed mxfp8 and
// fp8_e4m3; Qwen FP8-KV article's per-tensor symmetric FP8).
//
// Two kernels.  For long runs of tokens (prefill chunks), a wave takes one
// plane of 16 consecutive tokens of one kv head, so that what it writes lies
// in a few long runs of the tile (tokens of a 16-slot block are adjacent in
// it) and whole cache lines are written at once.  For a few tokens (a decode
// step's one per sequence), a wave takes one (token, kv head) and holds each
// row across all its lanes, so the time is a load, a short encode and the
// stores.  The encoders are in kvq_encode.hpp.
#include <hip/hip_runtime.h>

#include "kvq_encode.hpp"

namespace kvq {
namespace {

using namespace enc;

// One V item: the V rows of 16 consecutive tokens b0 .. b0 + 15 of one kv
// head, 4 tokens per row of 16 lanes.  When the slots from a = slot(b0) % 4
// slots earlier run on consecutively for 16 tokens, the item starts its
// window a tokens early instead, so every row holds one whole slab of the
// tile.  Item X writes exactly the tokens from its own window start up to
// the next item's (which it decides from the same slots the next item
// sees), so every token is written once: the rows take the first 16 and a
// second pass of row 0 the at most 3 left when the next window starts
// later than this one ends.  So a tile word is written either by one whole
// slab store or only by the atomics of the 4-bit per-token path.
template <int FMT, int D>
__device__ __forceinline__ void append_v_wave(uint8_t* __restrict__ pool, const uint16_t* __restrict__ v,
                                              int64_t T, const int32_t* __restrict__ slots, const Geometry& geo,
                                              float v_scale, int64_t vw, int lane) {
  const int64_t tg = vw / geo.H_kv;
  const int head = (int)(vw - tg * geo.H_kv);
  const int j = lane & 15, row = lane >> 4;
  const int64_t b0 = tg * 16;
  int64_t lo = b0, hi = b0 + 16;  // this item's tokens
  if constexpr (D == 256) {
    // lane l holds the slot of token b0 - 3 + l (l < 35; -1 outside [0, T)):
    // both windows are decided from these values with lane votes
    const int64_t tl = b0 - 3 + lane;
    const int sl = (lane < 35 && tl >= 0 && tl < T) ? slots[tl] : -1;
    // does every group of 4 tokens from lane l0 on fill one slab (slots
    // 4i, 4i + 1, 4i + 2, 4i + 3 of one page)?  Pages hold whole slabs, so
    // a run of slots that crosses pages still qualifies.
    auto slabs_from = [&](int l0) -> bool {
      const int k = lane - l0;
      const int f = __shfl(sl, l0 + (k & ~3));  // slot of the group's first token
      const bool in = k >= 0 && k < 16;
      return __all(!in || (sl >= 0 && (sl & 3) == (k & 3) && (sl >> 2) == (f >> 2)));
    };
    // the window shift of the item whose first token sits at lane l0 + 3
    auto window_shift = [&](int l0) -> int {
      const int s = __shfl(sl, l0 + 3);
      if (s < 0) return 0;
      const int a = s & 3;
      return slabs_from(l0 + 3 - a) ? a : 0;
    };
    lo = b0 - window_shift(0);
    hi = b0 + 16 - window_shift(16);
  }
  if (hi > T) hi = T;
  auto slot_of = [slots](int64_t tok) -> int { return slots[tok]; };
  v_row_group<FMT, D>(pool, v, slot_of, geo, v_scale, head, j, lo + 4 * row, lo, hi < lo + 16 ? hi : lo + 16);
  if (hi > lo + 16 && row == 0) v_row_group<FMT, D>(pool, v, slot_of, geo, v_scale, head, j, lo + 16, lo + 16, hi);
}

// One K item: the K rows of 16 consecutive tokens of one kv head.
template <int FMT, int D>
__device__ __forceinline__ void append_k_wave(uint8_t* __restrict__ pool, const uint16_t* __restrict__ k, int64_t T,
                                              const int32_t* __restrict__ slots, const Geometry& geo,
                                              float k_scale, int64_t kw, int lane) {
  const int q = lane & 3;
  const int64_t tg = kw / geo.H_kv;
  const int head = (int)(kw - tg * geo.H_kv);
  const int64_t token = tg * 16 + (lane >> 2);  // a whole quad shares it
  if (token >= T) return;
  uint32_t raw[D / 8];
  load_k_row<D>(raw, k + (token * geo.H_kv + head) * D + q * (D / 4));  // before the slot, so the loads overlap
  const int slot = slots[token];
  if (slot < 0) return;
  encode_k_row<FMT, D>(pool, raw, slot, geo, head, k_scale, q);
}

// Waves 2 i (K) and 2 i + 1 (V) cover 16 consecutive tokens of one kv head.
template <int FMT, int D>
__global__ __launch_bounds__(256) void append_kernel(uint8_t* __restrict__ pool, const uint16_t* __restrict__ k,
                                                     const uint16_t* __restrict__ v, int64_t T,
                                                     const int32_t* __restrict__ slots, Geometry geo,
                                                     float k_scale, float v_scale, int64_t items) {
  const int lane = threadIdx.x & 63;
  const int64_t it = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (it >= items) return;
  if ((it & 1) == 0) append_k_wave<FMT, D>(pool, k, T, slots, geo, k_scale, it >> 1, lane);
  else append_v_wave<FMT, D>(pool, v, T, slots, geo, v_scale, it >> 1, lane);
}

// Wave w of the grid encodes K and V of token w / H_kv, kv head w % H_kv.
template <int FMT, int D>
__global__ __launch_bounds__(256) void append_token_kernel(uint8_t* __restrict__ pool, const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v, int64_t T,
                                                           const int32_t* __restrict__ slots, Geometry geo,
                                                           float k_scale, float v_scale) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= T * geo.H_kv) return;  // whole waves
  const int64_t token = item / geo.H_kv;
  const int head = (int)(item - token * geo.H_kv);
  enc::TokenRow<D> rk, rv;  // loaded before the slot, so the three loads overlap
  enc::load_k_token<D>(rk, k + item * D, lane);
  enc::load_v_token<D>(rv, v + item * D, lane);
  const int slot = slots[token];
  if (slot < 0) return;
  enc::encode_k_token<FMT, D>(pool, rk, slot, geo, head, k_scale, lane);
  enc::encode_v_token<FMT, D>(pool, rv, slot, geo, head, v_scale, lane);
}

// Calls of at most this many tokens take append_token_kernel.
constexpr int64_t TOKEN_KERNEL_MAX_T = 256;

template <int FMT, int D>
hipError_t launch_append_t(uint8_t* pool, const uint16_t* k, const uint16_t* v, int64_t T, const int32_t* slots,
                           const Geometry& geo, float ks, float vs, hipStream_t stream) {
  if (T <= TOKEN_KERNEL_MAX_T) {
    const int64_t blocks = (T * geo.H_kv + 3) / 4;
    hipLaunchKernelGGL((append_token_kernel<FMT, D>), dim3((unsigned)blocks), dim3(256), 0, stream, pool, k, v, T,
                       slots, geo, ks, vs);
    return hipGetLastError();
  }
  const int64_t items = 2 * ((T + 15) / 16) * geo.H_kv;  // K and V of 16 tokens x 1 head each
  const int64_t blocks = (items + 3) / 4;
  hipLaunchKernelGGL((append_kernel<FMT, D>), dim3((unsigned)blocks), dim3(256), 0, stream, pool, k, v, T, slots,
                     geo, ks, vs, items);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(uint8_t* pool, const uint16_t* k, const uint16_t* v, int64_t T, const int32_t* slots,
                         const Geometry& geo, float ks, float vs, hipStream_t stream) {
#define KVQ_APPEND_CASE(F, DD) \
  if (geo.fmt == F && geo.D == DD) return launch_append_t<F, DD>(pool, k, v, T, slots, geo, ks, vs, stream);
  KVQ_APPEND_CASE(F_BF16, 128) KVQ_APPEND_CASE(F_BF16, 256)
  KVQ_APPEND_CASE(F_FP8_ROW, 128) KVQ_APPEND_CASE(F_FP8_ROW, 256)
  KVQ_APPEND_CASE(F_FP8_TENSOR, 128) KVQ_APPEND_CASE(F_FP8_TENSOR, 256)
  KVQ_APPEND_CASE(F_MXFP8, 128) KVQ_APPEND_CASE(F_MXFP8, 256)
  KVQ_APPEND_CASE(F_INT8_G64, 256) KVQ_APPEND_CASE(F_NVFP4_G16, 256) KVQ_APPEND_CASE(F_K8V4, 256)
  KVQ_APPEND_CASE(F_MXFP4, 256)
#undef KVQ_APPEND_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
