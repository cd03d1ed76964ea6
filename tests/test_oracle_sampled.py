"""Pins of the filtered accept/reject oracle (oracle/sampled.py): the
sampler's top-p / min-p filters and the acceptance rule on filtered
distributions, against what the definitions and the mathematics fix.

Sources: page "Decode is memory-bound ..." (trefon.com), section "Two things
that follow from the math" (production sampler: temperature 0.6, top-p 0.95,
min-p 0.05; expected acceptance = sum of min(p, q)) and section "Speculative
decoding" (the output follows the target distribution exactly); page
"Speculative decoding and early exit ..." (reactapp.top), listing
speculative_decode (the draft distribution from the draft's logits).
"""
import os

import numpy as np
import pytest
import scipy.stats

import oracle
from oracle import sampled as S

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                out.append([float(v) for v in line.split()])
    return out


def test_filters_hand_worked():
    z = np.array([2, 1, 1, 0, -1], np.float32)
    for r in _rows("sampler_filters.txt"):
        tp, mp, want = r[0], r[1], np.array(r[2:])
        got, keep, near, bad = S.filtered(z, 1.0, tp, mp)
        assert not bad and not near
        assert np.allclose(got, want, atol=6e-5), (tp, mp, got)
        assert np.array_equal(keep, want > 0)


def test_no_filter_is_the_softmax():
    rng = np.random.default_rng(1)
    z = rng.normal(0, 3, 1000).astype(np.float32)
    got, keep, _, _ = S.filtered(z, 0.6, 1.0, 0.0)
    ref = np.exp((z.astype(np.float64) - z.max()) / 0.6)
    assert np.allclose(got, ref / ref.sum(), rtol=1e-12, atol=0)
    assert keep.all()


def test_top_p_keeps_the_smallest_sufficient_prefix():
    # brute force over sorted prefixes on random distributions with ties
    rng = np.random.default_rng(2)
    for _ in range(200):
        z = np.round(rng.normal(0, 2, 40) * 2) / 2          # many ties
        p = np.exp(z - z.max())
        p /= p.sum()
        tp = float(np.float32(rng.uniform(0.05, 0.999)))
        got, keep, near, _ = S.filtered(z.astype(np.float32), 1.0, tp, 0.0)
        if near:
            continue
        vals = np.unique(z)[::-1]                # distinct values, descending
        cum = 0.0
        for v in vals:                           # keep whole tie groups until the mass reaches tp
            cum += p[z == v].sum()
            if cum >= tp:
                break
        assert np.array_equal(keep, z >= v)
        assert got[keep].sum() == pytest.approx(1.0, abs=1e-12)


def test_min_p_is_relative_to_the_top_token():
    rng = np.random.default_rng(3)
    z = rng.normal(0, 2, 500).astype(np.float32)
    for T in (0.6, 1.0, 1.7):
        for mp in (0.05, 0.2):
            got, keep, near, _ = S.filtered(z, T, 1.0, mp)
            p = np.exp((z.astype(np.float64) - z.max()) / T)
            p /= p.sum()
            if not near:
                assert np.array_equal(keep, p >= mp * p.max())


def test_unfiltered_matches_the_pinned_oracle():
    # with top_p = 1 and min_p = 0 the filtered pass is the plain pass: same
    # decisions as the C oracle given q = softmax(draft / T) (rows clear of
    # both oracles' near-threshold windows)
    rng = np.random.default_rng(4)
    B, K, V, T = 300, 4, 50, 0.8
    z = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    dl = (z[:, :K] + rng.normal(0, 1, (B, K, V))).astype(np.float32)
    q = np.exp((dl.astype(np.float64) - dl.max(-1, keepdims=True)) / np.float32(T))
    q /= q.sum(-1, keepdims=True)
    x = np.array([[rng.choice(V, p=q[b, i]) for i in range(K)] for b in range(B)], np.int32)
    L = rng.integers(0, K + 1, B).astype(np.int32)
    got = S.spec_accept_sampled(z, dl, x, L, T, T, 1.0, 0.0, seed=9, offset=3)
    oracle.build()
    ref = oracle.spec_accept(z, q.astype(np.float32), x, L, T, 9, 3)
    ok = ~got["near"] & (ref["near_acc"] < 0) & (ref["near_smp"] == 0)
    assert ok.mean() > 0.95
    assert np.array_equal(got["accepted"][ok], ref["accepted"][ok])
    assert np.array_equal(got["tokens"][ok], ref["tokens"][ok])


def _tiny(rounds, tp, mp, seed):
    rng = np.random.default_rng(seed)
    K, V, T = 3, 8, 0.9
    z1 = rng.normal(0, 1.5, (K + 1, V)).astype(np.float32)
    d1 = (z1[:K] + rng.normal(0, 1.0, (K, V))).astype(np.float32)
    qf = [S.filtered(d1[i], T, tp, mp)[0] for i in range(K)]
    x = np.stack([rng.choice(V, size=rounds, p=qf[i]) for i in range(K)], 1).astype(np.int32)
    z = np.broadcast_to(z1, (rounds, K + 1, V))
    d = np.broadcast_to(d1, (rounds, K, V))
    return z, d, x, z1, d1, qf, T


@pytest.mark.slow
@pytest.mark.parametrize("tp,mp", [(0.95, 0.05), (0.7, 0.0), (1.0, 0.3)])
def test_output_follows_the_filtered_target(tp, mp):
    # the acceptance rule on filtered distributions reproduces the filtered
    # target exactly: chi-square at every emitted position
    rounds = 20000
    z, d, x, z1, d1, qf, T = _tiny(rounds, tp, mp, seed=5)
    out = S.spec_accept_sampled(z, d, x, None, T, T, tp, mp, seed=11, offset=0)
    K = 3
    pvals = []
    for j in range(K + 1):
        pj = S.filtered(z1[j], T, tp, mp)[0]
        toks = out["tokens"][out["accepted"] >= j, j]
        cnt = np.bincount(toks, minlength=8)
        sup = pj > 0
        assert cnt[~sup].sum() == 0                   # never a filtered-out token
        if sup.sum() > 1:
            pvals.append(scipy.stats.chisquare(cnt[sup], pj[sup] * cnt.sum()).pvalue)
    assert min(pvals) > 1e-4 / len(pvals), pvals
    # acceptance at position 0 is the overlap sum of min(p', q')
    p0 = S.filtered(z1[0], T, tp, mp)[0]
    alpha = S.acceptance_overlap(p0, qf[0])
    acc0 = (out["accepted"] >= 1).mean()
    assert abs(acc0 - alpha) < 4 * np.sqrt(alpha * (1 - alpha) / rounds)


def test_positions_after_the_first_rejection_are_not_read():
    # the listing's break: a non-finite target logit after the first
    # rejection is never read; at or before it, the row is invalid.  The
    # draft side is validated for every drafted position.
    V, K, T = 12, 3, 1.0
    z = np.zeros((3, K + 1, V), np.float32)
    d = np.zeros((3, K, V), np.float32)
    z[:, 0, 5] = -40.0          # p'(5) ~ 0 at position 0 ...
    d[:, 0, 5] = 40.0           # ... where q' puts all its mass on token 5
    x = np.full((3, K), 5, np.int32)
    z[0, 2, 1] = np.nan         # after the rejection at 0: not read
    z[1, 0, 2] = np.inf         # at the rejected position: read
    d[2, 2, 3] = np.nan         # a draft distribution: validated for all drafts
    out = S.spec_accept_sampled(z, d, x, None, T, T, 1.0, 0.0, 9, 0)
    assert list(out["status"]) == [0, S.ROW_NONFINITE, S.ROW_NONFINITE]
    assert out["accepted"][0] == 0 and out["p_draft"][0, 0] < 1e-12
    assert np.all(out["p_draft"][0, 1:] == -1) and np.all(out["p_draft"][1:] == -1)


def _ambiguous_case():
    """V = 16, T = 1: p at position 0 = [0.5, 0.3, 0.15, 0.05/13 ...], so the
    mass above token 2 is 0.8 = top_p up to fp32 rounding of the logits (its
    top-p test is ambiguous); q = [0.6, 0.35/14 ..., 0.05 at token 2, ...]
    keeps every token firmly.  Position 1 is unambiguous (flat)."""
    V = 16
    p0 = np.full(V, 0.05 / 13)
    p0[:3] = [0.5, 0.3, 0.15]
    q0 = np.full(V, 0.35 / 14)
    q0[0], q0[2] = 0.6, 0.05
    z = np.zeros((1, 2, V), np.float32)
    z[0, 0] = np.log(p0)
    d = np.log(q0).astype(np.float32)[None, None, :]
    return z, d, float(np.float32(0.8))


def test_near_when_an_ambiguous_cut_decides_the_row():
    # x = token 2: kept, p'(2) = 0.15 / 0.95 > q'(2) = 0.05 and the draft is
    # accepted whatever u; dropped, p'(2) = 0 and it is rejected.  The
    # outcome hangs on the ambiguous cut, so the row is near.
    z, d, tp = _ambiguous_case()
    parts = S._filter_parts(z[0, 0], 1.0, tp, 0.0)
    assert len(parts[3]) == 1 and parts[3][0][0] == 0 and parts[3][0][1][2]
    o = S.spec_accept_sampled(z, d, np.array([[2]]), np.array([1]), 1.0, 1.0, tp, 0.0, 5, 0)
    assert o["near"][0]


def test_not_near_when_the_ambiguous_cut_does_not_matter():
    # x = token 0: p'(0) = 0.5 / 0.95 or 0.5 / 0.8, q'(0) = 0.6, so the
    # acceptance probability is 0.877 or 1; with u_acc below 0.8 the draft is
    # accepted either way and the bonus draw at the flat position 1 is
    # unambiguous: the row is pinned, and p'(0) is bounded by both values.
    z, d, tp = _ambiguous_case()
    off = next(o for o in range(200) if oracle.uniforms(5, o, 0, 0)[0] < 0.8)
    o = S.spec_accept_sampled(z, d, np.array([[0]]), np.array([1]), 1.0, 1.0, tp, 0.0, 5, off)
    assert not o["near"][0] and o["accepted"][0] == 1 and o["status"][0] == 0
    lo, hi, pd = o["p_draft_lo"][0, 0], o["p_draft_hi"][0, 0], o["p_draft"][0, 0]
    assert np.isclose(lo, 0.5 / 0.95, rtol=1e-6) and np.isclose(hi, 0.5 / 0.8, rtol=1e-6)
    assert lo <= pd <= hi
    # the earlier, coarser flag (any cut within 1e-6 at a position read) would
    # have excluded this row
    assert S.filtered(z[0, 0], 1.0, tp, 0.0)[2]


def test_near_when_an_ambiguous_min_p_test_decides_the_kept_set():
    # min-p at exactly p_2 / max p: token 2's min-p test is ambiguous; with
    # x = 2 in the draft the row's validity (ZERO_Q) hangs on it
    V = 8
    q0 = np.full(V, 0.3 / 6)
    q0[0], q0[2] = 0.6, 0.1
    d = np.log(q0).astype(np.float32)[None, None, :]
    z = np.zeros((1, 2, V), np.float32)
    mp = float(np.float32(np.exp(float(d[0, 0, 2]) - float(d[0, 0, 0]))))
    o = S.spec_accept_sampled(z, d, np.array([[2]]), np.array([1]), 1.0, 1.0, 1.0, mp, 5, 0)
    assert o["near"][0]
