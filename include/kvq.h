/*
 * kvq.h -- quantized paged KV cache and decode attention for AMD MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only; every call returns a kvq_status and
 * no C++ exception crosses the boundary.
 *
 * What the library computes comes from five web pages on KV-cache
 * quantization:
 *  - NInfer KV-cache quantization guide (m.xxqk.cn/news/579065): a paged KV
 *    cache with 64-token pages and independent K/V encodings; the formats
 *    BF16, INT8-G64, FP8-E4M3 row-256, NVFP4-G16 and the K8V4 profile, with
 *    their per-token byte counts at head_dim 256, and the normalized
 *    256-point Hadamard pre-rotation (section on the five formats); decode
 *    reads the whole cache every step, so stored bytes set its speed
 *    (section on why the cache is quantized).
 *  - TokenSpeed quantization article (gsyq.cn/news/441801), section on the
 *    --kv-cache-dtype options: fp8_e4m3 with unit scale, mxfp8 with one
 *    UE8M0 scale per 32 head_dim elements and 128-token blocks.
 *  - Qwen3.8-27B-NVFP4 FP8-KV article (lpnh.cn/news/1821634): per-tensor
 *    symmetric FP8 (kv_cache_scheme) and multi-token prediction (MTP).
 *
 * Ownership: the caller owns every buffer (pool, inputs, outputs, tables,
 * workspace).  The library never allocates or frees device memory and keeps
 * no mutable global state.  All work is enqueued asynchronously on the
 * caller's stream; nothing synchronizes.
 *
 * Errors: argument problems the host can see return KVQ_ERR_INVALID_ARGUMENT
 * or KVQ_ERR_UNSUPPORTED and enqueue nothing.  A workspace that is too small
 * returns KVQ_ERR_WORKSPACE_TOO_SMALL.  A failed kernel launch returns
 * KVQ_ERR_HIP.  Device-side contents (slot numbers, page-table entries,
 * sequence lengths) are preconditions the library does not check: they must
 * be in range.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARGUMENT = 1,
  KVQ_ERR_UNSUPPORTED = 2,
  KVQ_ERR_WORKSPACE_TOO_SMALL = 3,
  KVQ_ERR_HIP = 4
} kvq_status;

/* KV formats.  "K | V" planes; "rot" = pre-rotated by H/16 (256-point
 * Sylvester Hadamard) before quantization.  Bytes per token and kv head at
 * D = 256 in brackets (NInfer guide table; FP8_TENSOR and MXFP8 derived).
 *  KVQ_BF16        K: bf16 bits as given | V: IEEE fp16            [1024]
 *  KVQ_INT8_G64    int8 + fp16 scale per 64 values, K rot | same, V not rot   [528]
 *  KVQ_FP8_ROW     E4M3 + one fp16 scale per row | same            [516]
 *  KVQ_NVFP4_G16   E2M1 + UE4M3 scale per 16, rot | same, rot      [288]
 *                  (two-level: x / k_scale, x / v_scale first)
 *  KVQ_K8V4        K as FP8_ROW | V as NVFP4_G16 (rot)             [402]
 *  KVQ_MXFP8       E4M3 + UE8M0 scale per 32 | same                [528; 264 at D=128]
 *  KVQ_FP8_TENSOR  E4M3 of x / k_scale | E4M3 of x / v_scale       [512]
 *  KVQ_MXFP4       E2M1 + UE8M0 scale per 32, rot | same, rot      [272]
 * Scales are computed from the group's absolute maximum: fp16(amax/127),
 * fp16(amax/448), UE4M3(amax/6), and the OCP MX exponent
 * floor(log2 amax) - 8 (E4M3) or - 2 (E2M1); every element is then rounded to nearest-even from
 * x / scale computed in IEEE fp32 with the stored scale, saturating at the
 * format maximum.  The encoding is bit-exact and deterministic. */
typedef enum kvq_format {
  KVQ_BF16 = 0,
  KVQ_INT8_G64 = 1,
  KVQ_FP8_ROW = 2,
  KVQ_NVFP4_G16 = 3,
  KVQ_K8V4 = 4,
  KVQ_MXFP8 = 5,
  KVQ_FP8_TENSOR = 6,
  KVQ_MXFP4 = 7
} kvq_format;

/* One layer's KV cache.
 *  format        kvq_format value.
 *  head_dim      D: 128 or 256 for BF16, FP8_ROW, FP8_TENSOR, MXFP8;
 *                256 for INT8_G64, NVFP4_G16, K8V4, MXFP4 (the rotation is
 *                256-point).
 *  page_size     tokens per page: 64 or 128 (the pages use 64, and 128 for mxfp8).
 *  num_kv_heads  H_kv >= 1.
 *  num_pages     pages in the pool (> 0).
 *  k_scale, v_scale  per-tensor fp32 scales (> 0, finite) of the K / V
 *                planes that have one, ignored for the others:
 *                FP8_TENSOR: E4M3 of x / scale; 1.0 is the "unit scale".
 *                NVFP4_G16 (K and V) and K8V4 (V): the second level of
 *                two-level NVFP4, one fp32 scale per tensor above the
 *                16-value UE4M3 ones (a reading: the pages give NVFP4's
 *                16-value groups and leave any higher level open): the
 *                rotated row is divided by it in IEEE fp32 before its
 *                group scales are taken, and decoding multiplies it back.
 *                1.0 is the single-level format.
 */
typedef struct kvq_cache_desc {
  int32_t format;
  int32_t head_dim;
  int32_t page_size;
  int32_t num_kv_heads;
  int64_t num_pages;
  float k_scale;
  float v_scale;
} kvq_cache_desc;

/* Bytes of one page: H_kv head blocks of [K codes | K scales | V codes |
 * V scales], each plane padded to 128 bytes (no padding at the supported
 * shapes, so a page is exactly page_size x H_kv x the per-token bytes).
 * The per-token bytes are those of the NInfer guide's table of the five
 * formats at head_dim 256 (section on why the KV cache is quantized: BF16
 * 1024, INT8-G64 528, FP8 row-256 516, NVFP4-G16 288, K8V4 402 bytes per
 * token), and for the other formats the same count of codes plus scales:
 * FP8_TENSOR 512, MXFP8 528 (264 at head_dim 128), MXFP4 272.  The pages
 * are the guide's 64-token pages (128-token blocks for mxfp8, TokenSpeed
 * article, --kv-cache-dtype section).
 * The pool is num_pages consecutive pages; it must be 128-byte aligned.
 * Inside each plane, tokens are grouped in blocks of 16 stored in the order
 * the decode kernel's matrix-core lanes consume them; the index formulas are
 * spelled out in decode_attention_quant_amd/csrc/kvq_format.hpp.
 * Errors: KVQ_ERR_INVALID_ARGUMENT for a null pointer or a malformed
 * descriptor, KVQ_ERR_UNSUPPORTED for a (format, head_dim, page_size) the
 * library does not build. */
kvq_status kvq_page_bytes(const kvq_cache_desc* desc, size_t* bytes_per_page);

/* Quantize and store K/V rows (the write path; NInfer guide: every format
 * is written through its codec when a token enters the cache).
 *  pool          device, num_pages * page_bytes bytes, written.
 *  k_bf16, v_bf16  device, bf16 [num_tokens][num_kv_heads][head_dim].
 *  slot_mapping  device int32 [num_tokens]: page * page_size + offset;
 *                a negative entry skips that token.  Two tokens must not
 *                share a slot in one call.
 * Only the bits of the written slots change: 4-bit V codes share each byte
 * between two neighbouring slots, and the other slot's nibble is kept, also
 * when both are written by different calls in any order.  num_tokens == 0
 * is a no-op. */
kvq_status kvq_quantize_append(const kvq_cache_desc* desc, void* pool,
                               const void* k_bf16, const void* v_bf16,
                               int64_t num_tokens, const int32_t* slot_mapping,
                               hipStream_t stream);

/* Workspace bytes kvq_decode_attention and kvq_decode_step need for this
 * problem.  Decode reads every cached K/V of each sequence at every step
 * (NInfer guide, section on why the KV cache is quantized), so the read of
 * one (sequence, kv head) is split across workgroups; the workspace holds
 * each split's partial softmax state (running maximum, denominator and
 * unnormalized output per query row) until the cross-split reduce merges
 * them.  The size follows the library's own plan (kvq_decode_plan): as
 * many split workgroups as fit on the current device at once, fewer for
 * small problems.
 * Limits: batch <= 4096; (num_q_heads / num_kv_heads) * n_q <= 1024.
 * Errors as in kvq_decode_attention's argument checks; bytes must not be
 * NULL. */
kvq_status kvq_decode_workspace_size(const kvq_cache_desc* desc, int32_t batch, int32_t n_q,
                                     int32_t num_q_heads, int32_t max_pages_per_seq, size_t* bytes);

/* The same for a forced split: num_workgroups = 0 selects the library's
 * own plan (the size kvq_decode_workspace_size gives), a positive value that
 * many split workgroups, as passed to kvq_decode_split, kvq_decode_step_split
 * and kvq_decode_combine. */
kvq_status kvq_decode_workspace_size_for(const kvq_cache_desc* desc, int32_t batch, int32_t n_q,
                                         int32_t num_q_heads, int32_t max_pages_per_seq,
                                         int32_t num_workgroups, size_t* bytes);

/* Decode attention over the compressed cache (NInfer guide: each generated
 * token attends over every cached K/V; Qwen FP8-KV article: several query
 * tokens per step with MTP).
 *  q_bf16        device bf16 [batch][n_q][num_q_heads][head_dim].
 *  block_table   device int32 [batch][max_pages_per_seq]: logical page ->
 *                physical page; entries past a sequence's last page are not read.
 *  seq_lens      device int32 [batch]: cached tokens of each sequence,
 *                including its n_q newest ones (already appended).
 *  softmax_scale scale applied to q.k (e.g. 1/sqrt(head_dim)).
 *  out           device fp32 [batch][n_q][num_q_heads][head_dim], written.
 *  lse           device fp32 [batch][n_q][num_q_heads] (natural log of the
 *                softmax denominator plus the max score), or NULL.
 *  workspace     device, 256-byte aligned, >= kvq_decode_workspace_size bytes;
 *                its contents on entry do not matter.
 * Query token i of sequence b sits at position seq_lens[b] - n_q + i and
 * attends to positions 0..that one (causal among the new tokens); query
 * head h reads kv head h / (num_q_heads / num_kv_heads).  A query with no
 * visible key gets out = 0 and lse = -inf.  Results are deterministic for a
 * given device.
 * Value range: V is expanded to fp16 with its scale applied before the
 * P.V products, so the values written must satisfy |V| < 32768 for
 * INT8_G64, FP8_ROW, MXFP8 and MXFP4 (every decoded value then stays below
 * 33,000, inside fp16's range); BF16 stores V as fp16 (the format itself
 * overflows past 65504), and NVFP4_G16, K8V4 and FP8_TENSOR apply their
 * tensor scale to the output, so any finite V is fine there.  Past that
 * range results may be infinite or NaN. */
kvq_status kvq_decode_attention(const kvq_cache_desc* desc, const void* pool,
                                const void* q_bf16, int32_t batch, int32_t n_q,
                                int32_t num_q_heads, const int32_t* block_table,
                                int32_t max_pages_per_seq, const int32_t* seq_lens,
                                float softmax_scale, float* out, float* lse,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* kvq_decode_attention for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, and harnesses that
 * forbid allocation.  The workspace is a device array of
 * KVQ_NOALLOC_SCRATCH_BYTES inside the library (each GPU the library runs
 * on holds its own copy until the process ends); the caller still passes
 * the inputs and outputs.  The call allocates and frees nothing.  Its
 * first call on a device, with that device current, looks the array's
 * address up on that device (hipGetSymbolAddress) and keeps it.
 * Arguments, results and errors are those of kvq_decode_attention; a
 * problem whose planned workspace (kvq_decode_workspace_size) exceeds
 * KVQ_NOALLOC_SCRATCH_BYTES returns KVQ_ERR_WORKSPACE_TOO_SMALL and
 * enqueues nothing.  Every call on one GPU shares that GPU's array, so calls
 * that overlap on one GPU (on different streams, or from several threads
 * without ordering) race and must not be made; calls ordered on one stream
 * are fine (nothing in the array needs clearing between them). */
#define KVQ_NOALLOC_SCRATCH_BYTES (64 << 20)
kvq_status kvq_decode_attention_noalloc(const kvq_cache_desc* desc, const void* pool,
                                        const void* q_bf16, int32_t batch, int32_t n_q,
                                        int32_t num_q_heads, const int32_t* block_table,
                                        int32_t max_pages_per_seq, const int32_t* seq_lens,
                                        float softmax_scale, float* out, float* lse,
                                        hipStream_t stream);

/* One decode step with the append fused in (the decode-step variant of the
 * write path followed by attention; NInfer guide: every generated token
 * enters the cache through its codec and then attends over the whole
 * cache).  Equal to kvq_quantize_append of the n_q newest tokens of every
 * sequence followed by kvq_decode_attention, in one launch plus the
 * cross-split reduce: the split workgroup that owns a block stores the new
 * tokens that fall in it before reading it.
 *  pool          device, written (the new tokens' bytes) and read.
 *  k_new_bf16, v_new_bf16  device bf16 [batch][n_q][num_kv_heads][head_dim]:
 *                token i of sequence b is stored at position
 *                seq_lens[b] - n_q + i (skipped if negative), in the slot
 *                block_table[b][pos / page_size] * page_size + pos % page_size.
 *  The other arguments are those of kvq_decode_attention (seq_lens include
 *  the new tokens; the same workspace size).  Needs
 *  (num_q_heads / num_kv_heads) * n_q <= 16, else KVQ_ERR_UNSUPPORTED (call
 *  the two entry points instead).  The pool bytes and the results equal
 *  those of the two separate calls. */
kvq_status kvq_decode_step(const kvq_cache_desc* desc, void* pool, const void* k_new_bf16,
                           const void* v_new_bf16, const void* q_bf16, int32_t batch, int32_t n_q,
                           int32_t num_q_heads, const int32_t* block_table, int32_t max_pages_per_seq,
                           const int32_t* seq_lens, float softmax_scale, float* out, float* lse,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The two phases of kvq_decode_attention, for callers that merge partial
 * results themselves (e.g. several devices each holding a range of a long
 * sequence's pages) or time them apart.
 *
 * Schedule: the 16-token blocks of all (sequence b, kv head h) units, in
 * unit order u = b * num_kv_heads + h, with 24 positions between one unit
 * and the next (what a workgroup's visit to a further unit costs), form a
 * line of C = T + 24 (units - 1) positions, T the blocks: block i of unit u
 * sits at position cum_u + 24 u + i, cum_u the blocks of the units before u.
 * Of the ways = min(num_workgroups, ceil(C / lo)) split workgroups that get
 * work, lo = min(max(ceil(C / 256), 4), 128), workgroup w takes the blocks
 * at positions [floor(w C / ways), floor((w + 1) C / ways)); the others
 * take none.
 * kvq_decode_split writes, for every unit u and every workgroup w that
 * covers part of it, one partial per row r = i * G + j
 * (query token i, j-th query head of the group) into slot u + w:
 *   workspace = cum int32 [batch + 1] (cum[b] = num_kv_heads x blocks of
 *   sequences before b), then at the next 256-byte boundary (m, l) fp32
 *   [slots][rows][2], then at the next 256-byte boundary o fp32
 *   [slots][rows][head_dim]; slots = batch * num_kv_heads + num_workgroups,
 *   rows = G * n_q.  m is the running maximum in base-2 units of the scaled
 *   score, l the softmax denominator relative to it, o the unnormalized
 *   output in the original domain (the split phase rotates the partials of
 *   rotated V planes back: NVFP4_G16, K8V4, MXFP4).
 * kvq_decode_combine merges each unit's partials, normalizes and writes
 * out / lse exactly as kvq_decode_attention does; pass the same
 * num_workgroups (0 = planned) and flags to both.  It takes the sequences'
 * block counts from the workspace's cum table, which the split phase
 * wrote, so seq_lens must be the split's.
 * flags & KVQ_SPLIT_WRITE_WHOLE_UNITS: a unit held entirely by one split
 * workgroup is finished by the split phase (written to out / lse, which
 * kvq_decode_split then needs) and the combine skips it; this is what
 * kvq_decode_attention does.  Without it every unit leaves partials.
 * kvq_decode_split takes out / lse only for that flag (NULL otherwise).
 * flags & KVQ_SPLIT_Q_MXFP8 (KVQ_MXFP8 caches only, else
 * KVQ_ERR_UNSUPPORTED): a numerics mode of this library, not of the pages,
 * which quantize only the cache.  Each query row is first rounded to the
 * cache's own MXFP8 format (TokenSpeed article, --kv-cache-dtype section:
 * E4M3 values, one UE8M0 scale per 32 head_dim values, by the OCP MX rule
 * X = 2^(floor(log2 amax) - 8), round to nearest even, saturating at
 * 448 X), so that q . k runs on the block-scaled fp8 matrix cores with both
 * scales applied by the instruction; the result is the attention of the
 * rounded query (kvq_decode_combine accepts and ignores the flag).  It
 * applies to kvq_decode_split and kvq_decode_step_split. */
#define KVQ_SPLIT_WRITE_WHOLE_UNITS 1
#define KVQ_SPLIT_Q_MXFP8 2
kvq_status kvq_decode_split(const kvq_cache_desc* desc, const void* pool, const void* q_bf16,
                            int32_t batch, int32_t n_q, int32_t num_q_heads,
                            const int32_t* block_table, int32_t max_pages_per_seq,
                            const int32_t* seq_lens, float softmax_scale, int32_t num_workgroups,
                            int32_t flags, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);
kvq_status kvq_decode_combine(const kvq_cache_desc* desc, int32_t batch, int32_t n_q,
                              int32_t num_q_heads, int32_t max_pages_per_seq,
                              const int32_t* seq_lens, int32_t num_workgroups, int32_t flags,
                              const void* workspace, size_t workspace_bytes,
                              float* out, float* lse, hipStream_t stream);

/* The fused step's first phase: kvq_decode_split that also stores the new
 * tokens, as kvq_decode_step does (same arguments as kvq_decode_step, plus
 * num_workgroups and flags as in kvq_decode_split); finish with
 * kvq_decode_combine.  For callers that time or schedule the phases apart. */
kvq_status kvq_decode_step_split(const kvq_cache_desc* desc, void* pool, const void* k_new_bf16,
                                 const void* v_new_bf16, const void* q_bf16, int32_t batch, int32_t n_q,
                                 int32_t num_q_heads, const int32_t* block_table,
                                 int32_t max_pages_per_seq, const int32_t* seq_lens, float softmax_scale,
                                 int32_t num_workgroups, int32_t flags, float* out, float* lse,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Chunked-prefill causal attention over the compressed cache (NInfer guide:
 * a prefill chunk's tokens, once appended, attend over the cache causally;
 * the same quantity as kvq_decode_attention, for n_q up to a whole chunk).
 * Arguments, layouts and the causal rule are those of kvq_decode_attention:
 * query token i of sequence b sits at position seq_lens[b] - n_q + i (its
 * K/V already stored) and attends to positions 0 .. that one.  No
 * workspace: each (sequence, kv head) is not split; a workgroup takes 64
 * query rows (G * n_q rows per kv head) and walks the cache once for them.
 * Limits: G * n_q < 2^30; batch * num_kv_heads * ceil(G * n_q / 64) <= 2^30.
 * Errors as in kvq_decode_attention. */
kvq_status kvq_prefill_attention(const kvq_cache_desc* desc, const void* pool, const void* q_bf16,
                                 int32_t batch, int32_t n_q, int32_t num_q_heads,
                                 const int32_t* block_table, int32_t max_pages_per_seq,
                                 const int32_t* seq_lens, float softmax_scale, float* out, float* lse,
                                 hipStream_t stream);

/* The plan kvq_decode_attention uses for this problem on the current device:
 * split workgroups and partial slots.  The planned grid is one round of the
 * workgroups the device holds at once (CUs x resident workgroups per CU). */
kvq_status kvq_decode_plan(const kvq_cache_desc* desc, int32_t batch, int32_t n_q,
                           int32_t num_q_heads, int32_t max_pages_per_seq,
                           int32_t* num_workgroups, int32_t* num_slots);

#define KVQ_DEQUANT_STORED_DOMAIN 1

/* Decode one physical page to fp32 (a portable view of the cache; no extra
 * rounding: the llama.cpp FP8-KV article warns that quality depends on
 * avoiding additional rounding when caches move).
 *  k_out, v_out  device fp32 [num_kv_heads][page_size][head_dim], written.
 * flags & KVQ_DEQUANT_STORED_DOMAIN: return code x scale as stored (exact
 * in fp32 except FP8_TENSOR, which rounds the product once); otherwise
 * rotated planes are rotated back (H y / 16 in fp32).  Slots never written
 * decode whatever bytes they hold. */
kvq_status kvq_dequant_page(const kvq_cache_desc* desc, const void* pool, int64_t page,
                            int32_t flags, float* k_out, float* v_out, hipStream_t stream);

/* Static description of a status code. */
const char* kvq_status_string(kvq_status status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
