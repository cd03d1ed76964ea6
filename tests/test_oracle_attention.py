"""Pins of the verify-attention oracle (oracle/attention.py) against what the
definition and the mathematics fix, independent of any other implementation.

Definition: page "Speculative decoding and early exit ..." (reactapp.top),
section "Attention structure during decoding" (queries against the whole
key/value memory) and section "Speculative decoding: draft first, then
verify" (one target pass over K+1 positions); readings in the oracle's
header (causal within the verified block, grouped heads).
"""
import math

import numpy as np

from oracle import attention as A


def _rand(B, K, H, Hkv, d, S, seed):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(B, K + 1, H, d))
    k = rng.normal(size=(B, Hkv, S, d))
    v = rng.normal(size=(B, Hkv, S, d))
    return q, k, v


def test_brute_force_scalar_loops():
    B, K, H, Hkv, d, S = 2, 2, 4, 2, 8, 9
    q, k, v = _rand(B, K, H, Hkv, d, S, 1)
    ctx = [3, 5]
    L = [2, 1]
    sc = 0.3
    got = A.verify_attention(q, k, v, ctx, L, sc)
    for b in range(B):
        for i in range(K + 1):
            for h in range(H):
                if i > L[b]:
                    assert np.all(got[b, i, h] == 0.0)
                    continue
                g = h // (H // Hkv)
                T = ctx[b] + i + 1
                s = [sc * sum(q[b, i, h, e] * k[b, g, j, e] for e in range(d)) for j in range(T)]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = sum(w)
                for e in range(d):
                    o = sum(w[j] * v[b, g, j, e] for j in range(T)) / tot
                    assert abs(got[b, i, h, e] - o) < 1e-12


def test_zero_scale_is_the_mean_of_allowed_values():
    q, k, v = _rand(2, 3, 4, 4, 16, 40, 2)
    ctx = [10, 30]
    got = A.verify_attention(q, k, v, ctx, None, 0.0)
    for b in range(2):
        for i in range(4):
            T = ctx[b] + i + 1
            for h in range(4):
                assert np.allclose(got[b, i, h], v[b, h, :T].mean(0), rtol=0, atol=1e-13)


def test_causal_within_the_verified_block():
    q, k, v = _rand(1, 4, 2, 1, 8, 30, 3)
    ctx = [20]
    base = A.verify_attention(q, k, v, ctx, None, 0.35)
    for pos in range(20, 25):
        k2, v2 = k.copy(), v.copy()
        k2[0, 0, pos] += 3.0
        v2[0, 0, pos] -= 2.0
        got = A.verify_attention(q, k2, v2, ctx, None, 0.35)
        i_new = pos - 20            # the first query that sees position pos
        for i in range(5):
            same = np.allclose(got[0, i], base[0, i], rtol=0, atol=0)
            assert same == (i < i_new), (pos, i)


def test_dominant_key_selects_its_value():
    q, k, v = _rand(1, 1, 1, 1, 16, 12, 4)
    j = 7
    k[0, 0, j] = 80.0 * q[0, 0, 0] / np.dot(q[0, 0, 0], q[0, 0, 0])
    got = A.verify_attention(q, k, v, [11], [0], 1.0)
    assert np.allclose(got[0, 0, 0], v[0, 0, j], atol=1e-12)


def test_grouped_heads_equal_repeated_kv():
    q, k, v = _rand(2, 2, 8, 2, 8, 16, 5)
    ctx = [5, 9]
    got = A.verify_attention(q, k, v, ctx, [2, 1], 0.4)
    krep = np.repeat(k, 4, axis=1)
    vrep = np.repeat(v, 4, axis=1)
    ref = A.verify_attention(q, krep, vrep, ctx, [2, 1], 0.4)
    assert np.array_equal(got, ref)


def test_zero_drafts_is_plain_decode_attention():
    # L_b = 0: one query per sequence, as in the page's decode step
    q, k, v = _rand(3, 4, 2, 2, 8, 20, 6)
    ctx = [4, 11, 19]
    got = A.verify_attention(q, k, v, ctx, [0, 0, 0], 0.25)
    for b in range(3):
        assert np.all(got[b, 1:] == 0.0)
        for h in range(2):
            T = ctx[b] + 1
            s = 0.25 * (k[b, h, :T] @ q[b, 0, h])
            p = np.exp(s - s.max())
            p /= p.sum()
            assert np.allclose(got[b, 0, h], p @ v[b, h, :T], atol=1e-13)


def test_row_helper_and_byte_count():
    q, k, v = _rand(2, 3, 4, 2, 8, 24, 7)
    ctx = [6, 17]
    full = A.verify_attention(q, k, v, ctx, None, 0.5)
    for b, i, h in [(0, 0, 0), (1, 3, 3), (0, 2, 1)]:
        assert np.array_equal(A.verify_attention_row(q, k, v, ctx[b], b, i, h, 0.5), full[b, i, h])
    assert A.kv_bytes([6, 17], None, 3, 2, 8) == (10 + 21) * 2 * 8 * 2 * 2
