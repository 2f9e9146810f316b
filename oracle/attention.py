"""Quantize-append, page dequantization and fp64 decode attention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Decode attention has a plain definition: ordinary softmax attention over
the *decoded* cache.  Every decode step reads all cached K/V of the
sequence (NInfer guide, why-quantize section; Qwen FP8-KV article,
bandwidth section); this module computes that result directly in float64:

* token t of sequence b lives in page ``block_table[b][t // P]`` at slot
  ``t % P``;
* with n_q query tokens per sequence (the MTP article's several tokens per
  step), query i sits at position L_b - n_q + i and sees keys 0..that
  position (reading: causal among the new tokens; n_q = 1 sees all L_b);
* query head h reads kv head h // (H_q / H_kv) (reading: contiguous GQA
  groups);
* s_t = scale * q . k_t, o = sum_t softmax(s)_t v_t, lse = max + ln(sum);
  an empty key set gives o = 0 and lse = -inf (reading).
"""

import numpy as np

from . import formats as F
from . import layout as Lo
from .scalar import bf16_bits_to_f32


def quantize_append(geo, pool, k_bits, v_bits, slot_mapping, k_scale=1.0, v_scale=1.0):
    """Encode bf16 K/V rows [T][H_kv][D] and store them at their slots."""
    k_bits = np.asarray(k_bits, dtype=np.uint16)
    v_bits = np.asarray(v_bits, dtype=np.uint16)
    for h in range(geo.H_kv):
        kx = k_bits[:, h, :] if geo.kc == "bf16" else bf16_bits_to_f32(k_bits[:, h, :])
        vx = bf16_bits_to_f32(v_bits[:, h, :])
        kc, ks = F.encode_rows(geo.kc, geo.k_rot, kx, k_scale)
        vc, vs = F.encode_rows(geo.vc, geo.v_rot, vx, v_scale)
        Lo.write_rows(pool, geo, slot_mapping, h, kc, ks, vc, vs)


def decode_slots(geo, pool, slots, head, k_scale=1.0, v_scale=1.0, stored_domain=False):
    """float64 K and V rows of one kv head at the given slots."""
    kc, ks, vc, vs = Lo.read_rows(pool, geo, slots, head)
    K = F.decode_rows(geo.kc, geo.k_rot, kc, ks, k_scale, stored_domain)
    V = F.decode_rows(geo.vc, geo.v_rot, vc, vs, v_scale, stored_domain)
    return K, V


def dequant_page(geo, pool, page, k_scale=1.0, v_scale=1.0, stored_domain=True):
    """float64 K, V of one physical page: [H_kv][P][D] each."""
    slots = page * geo.P + np.arange(geo.P)
    K = np.empty((geo.H_kv, geo.P, geo.D))
    V = np.empty_like(K)
    for h in range(geo.H_kv):
        K[h], V[h] = decode_slots(geo, pool, slots, h, k_scale, v_scale, stored_domain)
    return K, V


def attend(q, K, V, scale, n_q):
    """Attention for one (sequence, kv head).

    q: [n_q, G, D] float64 (the G query heads sharing this kv head);
    K, V: [L, D] float64.  Returns out [n_q, G, D] and lse [n_q, G], both
    float64.
    """
    L = K.shape[0]
    nq, G, D = q.shape
    out = np.zeros((nq, G, D))
    lse = np.full((nq, G), -np.inf)
    for i in range(nq):
        p = L - n_q + i
        if p < 0:
            continue
        s = scale * (q[i] @ K[: p + 1].T)  # [G, p+1]
        m = s.max(axis=-1, keepdims=True)
        w = np.exp(s - m)
        z = w.sum(axis=-1, keepdims=True)
        out[i] = (w / z) @ V[: p + 1]
        lse[i] = (m + np.log(z))[:, 0]
    return out, lse


def quantize_query_mxfp8(q):
    """The query rounded to MXFP8 along head_dim, as float64 values.

    The pages quantize only the cache.  This is an optional mode of ours (a
    reading, not the pages' method): the query is put in the same MXFP8
    format as an MXFP8 cache's K (TokenSpeed article, ``--kv-cache-dtype``
    section: E4M3 elements, one UE8M0 scale per 32 head_dim elements), so
    that q . k is a product of two block-scaled FP8 operands.  Each row is
    encoded and decoded by the cache's own MXFP8 codec; a row's values are
    its bf16 values, unscaled (the softmax scale is applied to the product).
    """
    q = np.asarray(q, dtype=np.float64)
    rows = q.reshape(-1, q.shape[-1]).astype(np.float32)  # bf16 values: exact in float32
    codes, scales = F.encode_rows("e4m3_mx32", False, rows)
    return F.decode_rows("e4m3_mx32", False, codes, scales).reshape(q.shape)


def attention_ref(geo, pool, q_bits, block_table, seq_lens, softmax_scale, n_q,
                  k_scale=1.0, v_scale=1.0, only=None, q_mxfp8=False):
    """Decode attention over the paged pool.

    q_bits: bf16 bits [B][n_q][H_q][D].  Returns float64 out [B][n_q][H_q][D]
    and lse [B][n_q][H_q].  ``only`` optionally restricts the work to a list
    of (b, kv_head) pairs (other entries stay NaN) so that single outputs of
    very large problems can be computed one by one.  ``q_mxfp8`` replaces
    the query by ``quantize_query_mxfp8(q)`` first; nothing else changes.
    """
    q = bf16_bits_to_f32(np.asarray(q_bits, dtype=np.uint16)).astype(np.float64)
    if q_mxfp8:
        q = quantize_query_mxfp8(q)
    B, nq, H_q, D = q.shape
    G = H_q // geo.H_kv
    out = np.full((B, nq, H_q, D), np.nan)
    lse = np.full((B, nq, H_q), np.nan)
    pairs = only if only is not None else [(b, h) for b in range(B) for h in range(geo.H_kv)]
    for b, h in pairs:
        L = int(seq_lens[b])
        t = np.arange(L)
        slots = np.asarray(block_table[b], dtype=np.int64)[t // geo.P] * geo.P + t % geo.P
        K, V = decode_slots(geo, pool, slots, h, k_scale, v_scale)
        o, l = attend(q[b, :, h * G:(h + 1) * G, :], K, V, softmax_scale, n_q)
        out[b, :, h * G:(h + 1) * G, :] = o
        lse[b, :, h * G:(h + 1) * G] = l
    return out, lse
