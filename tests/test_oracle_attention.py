"""Pins of the oracle's decode attention over a rotated, quantised K/V cache
(oracle/hq_oracle.c, hqo_decode_attention), checked against things other than
the oracle itself:

- plain softmax attention in numpy on the unrotated K, V and q, with K and V
  taken back from the cache through scipy.linalg.hadamard (a library routine,
  not the oracle's Sylvester recursion): rotating q and K with the same
  orthogonal matrix keeps q.K^T ("哈特曼旋转，轻量级QAT，流式注意力" section 1),
  and the rotated weighted sum of V rotates back to the weighted sum of the
  unrotated V ("QuaRot：基于旋转的离群值抑制算法说明", principle);
- one cached token: the output is that token's dequantised V row rotated back,
  i.e. the (separately pinned) inverse path;
- a zero query: every weight is 1/tokens, the output is the mean of V;
- one dominant score: the output is that token's V.
"""
from __future__ import annotations

import numpy as np
import pytest
import scipy.linalg

from oracle import oracle as O


def _cache(rng, tokens, kv_heads, n, bits):
    qmax = 7 if bits == 4 else 127
    codes = rng.integers(-qmax, qmax + 1, size=(tokens * kv_heads, n))
    scales = (2.0 ** rng.integers(-6, 1, size=tokens * kv_heads)).astype(np.float32)
    return codes, scales


def _pack(codes, bits):
    if bits == 8:
        return codes.astype(np.int8).view(np.uint8)
    u = (codes & 0xF).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def _unrotate(rows, s, b):
    """Rows of the rotated space back to the input space: (y . H_b/sqrt(b)) * s,
    blockwise, with scipy's Hadamard matrix."""
    H = scipy.linalg.hadamard(b).astype(np.float64) / np.sqrt(b)
    n = rows.shape[1]
    out = np.empty_like(rows, dtype=np.float64)
    for k in range(0, n, b):
        out[:, k:k + b] = rows[:, k:k + b] @ H
    return out * s[None, :]


def _plain_attention(q, K, V):
    c = q @ K.T / np.sqrt(q.shape[-1])
    c = c - c.max(axis=-1, keepdims=True)
    w = np.exp(c)
    w /= w.sum(axis=-1, keepdims=True)
    return w @ V


@pytest.mark.parametrize("n,b,q_heads,kv_heads,tokens,bits", [
    (128, 128, 8, 2, 37, 4), (128, 128, 4, 4, 5, 8), (64, 16, 6, 3, 19, 4), (256, 128, 2, 1, 50, 4),
])
def test_matches_plain_attention_in_the_input_space(n, b, q_heads, kv_heads, tokens, bits):
    rng = np.random.default_rng(n + tokens)
    s = np.where(rng.integers(0, 2, n) == 1, 1, -1).astype(np.int8)
    q = rng.standard_normal((q_heads, n)).astype(np.float32)
    kc, ks = _cache(rng, tokens, kv_heads, n, bits)
    vc, vs = _cache(rng, tokens, kv_heads, n, bits)
    out = O.decode_attention(q, O.F32, kv_heads, b, s, _pack(kc, bits), ks, _pack(vc, bits), vs,
                             O.F32, bits)
    # the cache rows in the input space
    K = _unrotate(kc * ks[:, None].astype(np.float64), s, b)
    V = _unrotate(vc * vs[:, None].astype(np.float64), s, b)
    group = q_heads // kv_heads
    for h in range(q_heads):
        kh = h // group
        rows = np.arange(tokens) * kv_heads + kh
        ref = _plain_attention(q[h].astype(np.float64), K[rows], V[rows])
        np.testing.assert_allclose(out[h], ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_single_token_is_the_inverse_path():
    rng = np.random.default_rng(3)
    n, b, kv_heads, bits = 128, 128, 2, 4
    s = np.where(rng.integers(0, 2, n) == 1, 1, -1).astype(np.int8)
    q = rng.standard_normal((4, n)).astype(np.float32) * 10
    kc, ks = _cache(rng, 1, kv_heads, n, bits)
    vc, vs = _cache(rng, 1, kv_heads, n, bits)
    out = O.decode_attention(q, O.F32, kv_heads, b, s, _pack(kc, bits), ks, _pack(vc, bits), vs,
                             O.F32, bits)
    inv = O.dequant_rotate_inv(_pack(vc, bits), vs, O.F32, b, s, bits, n)
    for h in range(4):
        np.testing.assert_allclose(out[h], inv[h // 2], rtol=0, atol=1e-13)


def test_zero_query_averages_v():
    rng = np.random.default_rng(4)
    n, b, kv_heads, tokens, bits = 64, 64, 1, 9, 8
    s = np.where(rng.integers(0, 2, n) == 1, 1, -1).astype(np.int8)
    q = np.zeros((3, n), dtype=np.float32)
    kc, ks = _cache(rng, tokens, kv_heads, n, bits)
    vc, vs = _cache(rng, tokens, kv_heads, n, bits)
    out = O.decode_attention(q, O.F32, kv_heads, b, s, _pack(kc, bits), ks, _pack(vc, bits), vs,
                             O.F32, bits)
    inv = O.dequant_rotate_inv(_pack(vc, bits), vs, O.F32, b, s, bits, n)
    np.testing.assert_allclose(out, np.broadcast_to(inv.mean(axis=0), out.shape), rtol=0,
                               atol=1e-13)


def test_dominant_score_selects_one_token():
    # q aligned with one cached key (in the rotated space) and far larger than
    # the rest: softmax puts all weight on that token
    rng = np.random.default_rng(5)
    n, b, tokens, bits = 128, 128, 12, 4
    s = np.where(rng.integers(0, 2, n) == 1, 1, -1).astype(np.int8)
    kc, ks = _cache(rng, tokens, 1, n, bits)
    vc, vs = _cache(rng, tokens, 1, n, bits)
    pick = 7
    kc[pick] = 7
    ks[pick] = 1.0
    K = _unrotate(kc * ks[:, None].astype(np.float64), s, b)
    q = (K[pick] * 200.0).astype(np.float32)[None, :]
    out = O.decode_attention(q, O.F32, 1, b, s, _pack(kc, bits), ks, _pack(vc, bits), vs,
                             O.F32, bits)
    inv = O.dequant_rotate_inv(_pack(vc, bits), vs, O.F32, b, s, bits, n)
    np.testing.assert_allclose(out[0], inv[pick], rtol=0, atol=1e-9)


def test_rejects_bad_arguments():
    q = np.zeros((3, 128), dtype=np.float32)
    s = np.ones(128, dtype=np.int8)
    c = np.zeros((4, 64), dtype=np.uint8)
    sc = np.ones(4, dtype=np.float32)
    with pytest.raises(ValueError):   # 3 query heads over 2 kv heads
        O.decode_attention(q, O.F32, 2, 128, s, c, sc, c, sc, O.F32, 4)
    with pytest.raises(ValueError):   # bits
        O.decode_attention(q, O.F32, 1, 128, s, c, sc, c, sc, O.F32, 3)
