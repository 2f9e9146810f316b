"""Pins for the oracle's fp64 decode attention over the paged pool (CPU only)."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A, layout as Lo, formats as F, scalar as S


def _bf16(x):
    return (torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
            .view(torch.int16).numpy().view(np.uint16))


def _case(fmt, lens, H_q, H_kv, n_q, P, seed, D=256, perm=True):
    rng = np.random.default_rng(seed)
    geo = Lo.Geometry(fmt, D, P, H_kv)
    npg = [max(1, -(-L // P)) for L in lens]
    total = sum(npg)
    order = rng.permutation(total)  # drawn either way: same stream below
    if not perm:
        order = np.arange(total)
    bt = np.zeros((len(lens), max(npg)), dtype=np.int64)
    k = 0
    for b, n in enumerate(npg):
        bt[b, :n] = order[k:k + n]
        k += n
    pool = np.full(total * geo.page_bytes, 0xFF, dtype=np.uint8)
    K = rng.standard_normal((sum(lens), H_kv, D)).astype(np.float32)
    K[..., [3, 50]] *= 20
    V = rng.standard_normal((sum(lens), H_kv, D)).astype(np.float32)
    slots = np.concatenate([bt[b, np.arange(L) // P] * P + np.arange(L) % P for b, L in enumerate(lens)]).astype(np.int64)
    kb, vb = _bf16(K), _bf16(V)
    A.quantize_append(geo, pool, kb, vb, slots, 0.1, 0.1)
    q = _bf16(rng.standard_normal((len(lens), n_q, H_q, D)))
    return geo, pool, q, bt, np.array(lens), kb, vb


def _brute(geo, pool, q_bits, bt, lens, scale, n_q, b, i, h):
    """Scalar loops: one output row, straight from the definition."""
    G = q_bits.shape[2] // geo.H_kv
    hk = h // G
    L = int(lens[b])
    pos = L - n_q + i
    qv = S.bf16_bits_to_f32(q_bits[b, i, h]).astype(np.float64)
    if pos < 0:
        return np.zeros(geo.D), -math.inf
    ks, vs = [], []
    for t in range(pos + 1):
        slot = int(bt[b, t // geo.P]) * geo.P + t % geo.P
        Kt, Vt = A.decode_slots(geo, pool, [slot], hk, 0.1, 0.1)
        ks.append(Kt[0])
        vs.append(Vt[0])
    s = [scale * sum(qv[d] * kt[d] for d in range(geo.D)) for kt in ks]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    z = sum(w)
    o = [sum(w[t] * vs[t][d] for t in range(len(w))) / z for d in range(geo.D)]
    return np.array(o), m + math.log(z)


@pytest.mark.parametrize("fmt,n_q", [(0, 1), (2, 1), (1, 4), (3, 1), (4, 4)])
def test_attention_equals_brute_force_loops(fmt, n_q):
    lens = [130, 65, 3]
    geo, pool, q, bt, L, _, _ = _case(fmt, lens, 4, 2, n_q, 64, 31 + fmt)
    scale = 1 / 16
    out, lse = A.attention_ref(geo, pool, q, bt, L, scale, n_q, 0.1, 0.1)
    for b, i, h in [(0, n_q - 1, 3), (1, 0, 0), (2, 0, 2)]:
        o, l = _brute(geo, pool, q, bt, L, scale, n_q, b, i, h)
        assert np.allclose(out[b, i, h], o, rtol=1e-12, atol=1e-12)
        assert (l == lse[b, i, h]) or abs(l - lse[b, i, h]) < 1e-10


def test_softmax_rows_sum_to_one_and_lse_consistent():
    geo, pool, q, bt, L, _, _ = _case(2, [200], 4, 2, 1, 64, 40)
    qv = S.bf16_bits_to_f32(q).astype(np.float64)
    slots = bt[0, np.arange(200) // 64] * 64 + np.arange(200) % 64
    K, V = A.decode_slots(geo, pool, slots, 0, 0.1, 0.1)
    s = (qv[0, 0, :2] @ K.T) / 16
    out, lse = A.attend(qv[0, :, :2], K, V, 1 / 16, 1)
    w = np.exp(s - lse[0][:, None])
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-12)
    assert np.allclose(w @ V, out[0], atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(41)
    D = 256
    V = rng.standard_normal((50, D))
    q = rng.standard_normal((1, 3, D))
    # all keys equal -> the mean of the values
    K = np.tile(rng.standard_normal(D), (50, 1))
    o, _ = A.attend(q, K, V, 0.1, 1)
    assert np.allclose(o[0], V.mean(axis=0)[None].repeat(3, 0), atol=1e-12)
    # one key -> its value, lse = its score
    o, l = A.attend(q, K[:1], V[:1], 0.1, 1)
    assert np.allclose(o[0], V[0][None].repeat(3, 0), atol=1e-15)
    assert np.allclose(l[0], 0.1 * q[0] @ K[0], atol=1e-12)
    # one score ahead by more than 50 -> that value
    K = rng.standard_normal((50, D)) * 0.01
    K[17] = q[0, 0] * 10
    o, _ = A.attend(q[:, :1], K, V, 1.0, 1)
    assert np.allclose(o[0, 0], V[17], atol=1e-15)


def test_bf16_format_equals_textbook_dense_attention():
    """BF16 format: K stored bitwise, V as fp16; attention over it equals
    torch's CPU float64 scaled_dot_product_attention with no paging."""
    lens = [150]
    geo, pool, q, bt, L, kb, vb = _case(0, lens, 4, 2, 1, 64, 42)
    out, _ = A.attention_ref(geo, pool, q, bt, L, 1 / 16, 1)
    Kd = torch.from_numpy(S.bf16_bits_to_f32(kb).astype(np.float64))  # [T, H_kv, D]
    Vd = torch.from_numpy(S.bf16_bits_to_f32(vb).astype(np.float16).astype(np.float64))
    Q = torch.from_numpy(S.bf16_bits_to_f32(q).astype(np.float64))[0, 0]  # [H_q, D]
    Kr = Kd.repeat_interleave(2, dim=1).permute(1, 0, 2)  # [H_q, T, D]
    Vr = Vd.repeat_interleave(2, dim=1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(Q[:, None], Kr, Vr, scale=1 / 16)[:, 0]
    assert np.allclose(out[0, 0], ref.numpy(), atol=1e-12)


def test_page_permutation_invariance():
    a = _case(3, [100, 40], 4, 2, 1, 64, 43, perm=False)
    b = _case(3, [100, 40], 4, 2, 1, 64, 43, perm=True)
    oa, la = A.attention_ref(a[0], a[1], a[2], a[3], a[4], 1 / 16, 1)
    ob, lb = A.attention_ref(b[0], b[1], b[2], b[3], b[4], 1 / 16, 1)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_mtp_is_causal_among_new_tokens():
    geo, pool, q, bt, L, _, _ = _case(5, [300], 2, 2, 4, 128, 44, D=128)
    out4, lse4 = A.attention_ref(geo, pool, q, bt, L, 0.09, 4)
    for i in range(4):
        o1, l1 = A.attention_ref(geo, pool, q[:, i:i + 1], bt, np.array([300 - 3 + i]), 0.09, 1)
        assert np.allclose(out4[:, i], o1[:, 0], atol=1e-14)


def test_empty_sequence_and_short_mtp():
    geo, pool, q, bt, _, _, _ = _case(2, [5], 4, 2, 4, 64, 45)
    out, lse = A.attention_ref(geo, pool, q, bt, np.array([0]), 1 / 16, 4)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    out, lse = A.attention_ref(geo, pool, q, bt, np.array([2]), 1 / 16, 4)
    assert np.all(out[0, :2] == 0) and np.all(np.isfinite(lse[0, 2:]))
