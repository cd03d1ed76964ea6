"""spec_accept_sampled on the GPU against the filtered oracle
(oracle/sampled.py): decisions, emitted tokens and status bits match exactly
on every row whose decisions (filter cut, acceptance test, draw) lie clear of
their thresholds by 1e-6; p'(x) within 1e-5 relative.

Definition: page "Decode is memory-bound ..." (trefon.com), section "Two
things that follow from the math" (production sampler: temperature 0.6,
top-p 0.95, min-p 0.05) and section "Speculative decoding" (acceptance rule);
page "Speculative decoding and early exit ..." (reactapp.top), listing
speculative_decode (draft distribution from the draft's logits).
"""
import numpy as np
import pytest
import scipy.stats
import torch

import oracle
import speculative_decoding_verification_accept_amd as sv
from oracle import sampled as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()
    oracle.set_mutation(0)
    sv.load_library()


def make_inputs(B, K, V, *, std, noise, T, top_p, min_p, seed, bf16=False, ragged=False):
    """Target logits ~ N(0, std^2), draft logits = target + N(0, noise^2)
    (rounded to the dtype), draft tokens drawn from the oracle's filtered
    draft distribution q' (the drafter's own sampling)."""
    rng = np.random.default_rng(seed)
    z = rng.normal(0, std, (B, K + 1, V)).astype(np.float32)
    d = (z[:, :K] + rng.normal(0, noise, (B, K, V))).astype(np.float32)
    if bf16:
        z = torch.from_numpy(z).to(torch.bfloat16).float().numpy()
        d = torch.from_numpy(d).to(torch.bfloat16).float().numpy()
    x = np.zeros((B, K), np.int32)
    for b in range(B):
        for i in range(K):
            q = S.filtered(d[b, i], T, float(np.float32(top_p)), float(np.float32(min_p)))[0]
            x[b, i] = rng.choice(V, p=q / q.sum())
    L = rng.integers(0, K + 1, B).astype(np.int32) if ragged else np.full(B, K, np.int32)
    return z, d, x, L


def run(z, d, x, L, *, T, Td=None, top_p, min_p, seed, offset, bf16=False, row_base=0, label=""):
    Td = T if Td is None else Td
    dt = torch.bfloat16 if bf16 else torch.float32
    dev = torch.device("cuda:0")
    B, K1, V = z.shape
    print(f"[spec_accept_sampled] {label} B={B} K={K1 - 1} V={V} {dt} T={T} top_p={top_p} min_p={min_p}",
          flush=True)
    zt = torch.from_numpy(np.ascontiguousarray(z)).to(dt).to(dev)
    dtt = torch.from_numpy(np.ascontiguousarray(d)).to(dt).to(dev)
    res = sv.accept_sampled(zt, dtt, torch.from_numpy(x).to(dev),
                            None if L is None else torch.from_numpy(L).to(dev), temperature=T,
                            draft_temperature=Td, top_p=top_p, min_p=min_p, seed=seed,
                            offset=offset, row_base=row_base)
    torch.cuda.synchronize()
    g = {k: getattr(res, k).cpu().numpy() for k in ("tokens", "accepted", "p_draft", "status")}
    o = S.spec_accept_sampled(z, d, x, L, T, Td, top_p, min_p, seed, offset, row_base=row_base)
    return g, o


def compare(g, o, label, max_near=0.05):
    near = o["near"]
    ok = ~near
    assert near.mean() <= max_near, (label, near.mean())
    st_g = g["status"]
    assert np.array_equal(st_g[ok], o["status"][ok]), (label, np.nonzero(st_g[ok] != o["status"][ok]))
    assert np.array_equal(g["accepted"][ok], o["accepted"][ok]), label
    assert np.array_equal(g["tokens"][ok], o["tokens"][ok]), label
    # p'(x) within 1e-5 of the oracle's, or of the range it spans when a
    # filter decision is ambiguous without changing the outcome
    m = ok[:, None] & (o["p_draft"] >= 0)
    pg = g["p_draft"][m].astype(np.float64)
    lo, hi = o["p_draft_lo"][m], o["p_draft_hi"][m]
    assert np.all((pg >= lo * (1 - 1e-5) - 1e-12) & (pg <= hi * (1 + 1e-5) + 1e-12)), label
    assert np.all(g["p_draft"][~(o["p_draft"] >= 0) & ok[:, None]] == -1.0)
    return dict(rows=len(ok), near=int(near.sum()), accepted_mean=float(o["accepted"][ok].mean()))


@pytest.mark.parametrize("top_p,min_p", [(0.95, 0.05), (1.0, 0.0), (0.9, 0.0), (1.0, 0.1), (0.5, 0.02)])
def test_mid_fp32(top_p, min_p):
    z, d, x, L = make_inputs(8, 4, 32000, std=3.0, noise=1.0, T=0.6, top_p=top_p, min_p=min_p, seed=2)
    g, o = run(z, d, x, L, T=0.6, top_p=top_p, min_p=min_p, seed=7, offset=1, label="mid")
    print(compare(g, o, ("mid", top_p, min_p)))


def test_many_rows_bf16_ragged():
    z, d, x, L = make_inputs(48, 5, 20000, std=2.0, noise=1.0, T=0.8, top_p=0.95, min_p=0.05,
                             seed=3, bf16=True, ragged=True)
    g, o = run(z, d, x, L, T=0.8, top_p=0.95, min_p=0.05, seed=11, offset=4, bf16=True, label="ragged")
    st = compare(g, o, "ragged")
    print(st)
    assert np.any(o["accepted"] < L) and np.any(o["accepted"] == L)


def test_at_scale_vocab_bf16():
    # the at-scale vocabulary (V = 128256, bf16), a batch the oracle finishes quickly
    z, d, x, L = make_inputs(6, 7, 128256, std=3.0, noise=1.5, T=0.8, top_p=0.95, min_p=0.05,
                             seed=4, bf16=True, ragged=True)
    g, o = run(z, d, x, L, T=0.8, top_p=0.95, min_p=0.05, seed=5, offset=9, bf16=True, label="scale")
    print(compare(g, o, "scale"))


def test_bench_size_sampled_rows():
    # the benchmark's launch: B = 64, K = 7, V = 128256 bf16, T = 0.8, top-p
    # 0.95, min-p 0.05, its own input recipe; the rows are independent (the
    # Philox stream of row b is that of global row b), so the oracle checks a
    # sample of them one by one with row_base = b
    from speculative_decoding_verification_accept_amd import workloads
    dev = torch.device("cuda:0")
    z, d, x, L = workloads.sampled_accept_device(4000, dev)
    B, K1, V = z.shape
    print(f"[spec_accept_sampled] bench size B={B} K={K1 - 1} V={V}", flush=True)
    res = sv.accept_sampled(z, d, x, L, temperature=0.8, top_p=0.95, min_p=0.05, seed=77, offset=0)
    torch.cuda.synchronize()
    g = {k: getattr(res, k).cpu().numpy() for k in ("tokens", "accepted", "p_draft", "status")}
    zh, dh = z.float().cpu().numpy(), d.float().cpu().numpy()
    xh, Lh = x.cpu().numpy(), L.cpu().numpy()
    rows = sorted({0, B - 1, *np.random.default_rng(7).integers(0, B, 16).tolist()})
    gs = {k: v[rows] for k, v in g.items()}
    parts = [S.spec_accept_sampled(zh[b:b + 1], dh[b:b + 1], xh[b:b + 1], Lh[b:b + 1], 0.8, 0.8, 0.95, 0.05, 77, 0,
                                   row_base=b) for b in rows]
    o = {k: np.concatenate([p_[k] for p_ in parts]) for k in parts[0]}
    st = compare(gs, o, "bench size", max_near=0.1)
    print(st)
    assert st["rows"] >= 12


@pytest.mark.parametrize("bf16", [False, True])
def test_top_p_alone_peaked(bf16):
    # top-p alone on peaked distributions (a few dozen dominant tokens per
    # position), the shape of real next-token distributions
    rng = np.random.default_rng(23 + bf16)
    B, K, V, T, tp = 8, 3, 50000, 0.9, 0.8
    z = rng.normal(0, 2.0, (B, K + 1, V))
    for b in range(B):
        for i in range(K + 1):
            z[b, i, rng.choice(V, 30, replace=False)] += rng.uniform(8.0, 12.0, 30)
    z = z.astype(np.float32)
    d = (z[:, :K] + rng.normal(0, 0.7, (B, K, V))).astype(np.float32)
    if bf16:
        z = torch.from_numpy(z).to(torch.bfloat16).float().numpy()
        d = torch.from_numpy(d).to(torch.bfloat16).float().numpy()
    x = np.zeros((B, K), np.int32)
    for b in range(B):
        for i in range(K):
            q = S.filtered(d[b, i], T, float(np.float32(tp)), 0.0)[0]
            x[b, i] = rng.choice(V, p=q / q.sum())
    g, o = run(z, d, x, rng.integers(0, K + 1, B).astype(np.int32), T=T, top_p=tp, min_p=0.0, seed=8, offset=2,
               bf16=bf16, label="top-p alone, peaked")
    print(compare(g, o, ("top-p alone", bf16), max_near=0.13))


def test_flat_distribution_deep_top_p_cut():
    # small logit spread: the top-p cut falls deep in the vocabulary, in a
    # crossing bin with many entries.  Distinct logits then sit ~3e-5 of mass
    # apart, so a cut within the 1e-6 window of top_p is not rare (~7% per
    # distribution); a row is excluded only when taking such a cut the other
    # way changes its outcome.
    z, d, x, L = make_inputs(16, 3, 30000, std=0.3, noise=0.1, T=1.0, top_p=0.9, min_p=0.0, seed=6)
    g, o = run(z, d, x, L, T=1.0, top_p=0.9, min_p=0.0, seed=3, offset=0, label="flat")
    st = compare(g, o, "flat", max_near=0.13)
    print(st)
    assert st["rows"] - st["near"] >= 14


def test_different_draft_temperature_and_edges():
    for (B, K, V, bf16) in [(5, 3, 7, False), (4, 0, 500, False), (3, 2, 1, False), (6, 3, 8195, True),
                            (4, 2, 16384 + 5, False)]:
        z, d, x, L = make_inputs(B, K, V, std=2.0, noise=0.5, T=0.7, top_p=0.9, min_p=0.05,
                                 seed=100 + V % 13, bf16=bf16)
        # the drafter samples at its own temperature
        rng = np.random.default_rng(V)
        for b in range(B):
            for i in range(K):
                q = S.filtered(d[b, i], 1.3, 0.9, float(np.float32(0.05)))[0]
                x[b, i] = rng.choice(V, p=q / q.sum())
        g, o = run(z, d, x, L, T=0.7, Td=1.3, top_p=0.9, min_p=0.05, seed=2, offset=5, bf16=bf16,
                   label=f"edge {B},{K},{V}")
        print(compare(g, o, ("edge", B, K, V), max_near=0.34))


def _single_pass_rows(V, K, rng):
    """Rows that stress the statistics pass in every filter mode (the one
    pass of min-p, the general passes without it): a rising ramp
    (the reference max grows every round), a jump of 600 mid-row (the round
    is summed again against the new reference), a -inf prefix (no finite
    reference for several rounds), a row that is -inf but for its last
    entries, flat logits (every entry passes min-p: more entries than the
    collection holds, so the general passes run), a NaN inside a -inf
    prefix, a +inf mid-row, and a plain Gaussian row."""
    B = 8
    z = rng.normal(0, 2.0, (B, K + 1, V))
    z[0] = np.linspace(-5.0, 30.0, V) + rng.normal(0, 0.1, (K + 1, V))
    z[1, :, : V // 2] = rng.normal(-600.0, 1.0, (K + 1, V // 2))
    z[2, :, : (2 * V) // 5] = -np.inf
    z[3, :, :-5] = -np.inf
    z[4] = rng.normal(0, 0.001, (K + 1, V))
    z[5, :, : V // 4] = -np.inf
    z[5, 0, 10] = np.nan
    z[6, 0, V // 2] = np.inf
    z = z.astype(np.float32)
    d = z[:, :K].copy()
    fin = np.isfinite(d)
    d[fin] += rng.normal(0, 0.5, int(fin.sum())).astype(np.float32)
    return z, d


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("top_p,mp", [(1.0, 0.05), (0.9, 0.05), (0.9, 0.0), (1.0, 0.0)])
def test_one_pass_edges(bf16, top_p, mp):
    V, K, T = 20000 + (3 if not bf16 else 0), 2, 0.8
    rng = np.random.default_rng(41 + bf16)
    z, d = _single_pass_rows(V, K, rng)
    if bf16:
        z = torch.from_numpy(z).to(torch.bfloat16).float().numpy()
        d = torch.from_numpy(d).to(torch.bfloat16).float().numpy()
    B = z.shape[0]
    x = np.zeros((B, K), np.int32)
    for b in range(B):
        for i in range(K):
            q = S.filtered(d[b, i], T, float(np.float32(top_p)), float(np.float32(mp)))[0]
            if q is not None:
                x[b, i] = rng.choice(V, p=q / q.sum())
    g, o = run(z, d, x, np.full(B, K, np.int32), T=T, top_p=top_p, min_p=mp, seed=5, offset=1, bf16=bf16,
               label=f"one-pass edges top_p={top_p} min_p={mp}")
    assert o["status"][5] == S.ROW_NONFINITE and o["status"][6] == S.ROW_NONFINITE
    assert (g["status"][5] & S.ROW_NONFINITE) and (g["status"][6] & S.ROW_NONFINITE)
    assert not np.any(o["status"][[0, 1, 2, 3, 4, 7]])
    print(compare(g, o, ("one-pass edges", bf16, top_p, mp), max_near=0.13))


def test_status_bits():
    z, d, x, L = make_inputs(8, 3, 9000, std=2.0, noise=1.0, T=1.0, top_p=0.95, min_p=0.05, seed=8)
    z[0, 0, 17] = np.nan                  # target position 0: always read
    z[6, 2, 50] = np.nan                  # read only if drafts 0 and 1 are accepted
    d[1, 2, 40] = np.inf
    x[2, 0] = 9000                        # out of range
    L[3] = 4                              # > K
    q = S.filtered(d[4, 1], 1.0, 0.95, float(np.float32(0.05)))[1]
    x[4, 1] = int(np.nonzero(~q)[0][0])   # outside the draft's kept set
    z[5, 3, 100] = np.nan                 # past L below: not read
    L[5] = 2
    g, o = run(z, d, x, L, T=1.0, top_p=0.95, min_p=0.05, seed=1, offset=0, label="status")
    assert list(o["status"][:6]) == [1, 1, 2, 4, 8, 0]
    assert list(g["status"][:6]) == [1, 1, 2, 4, 8, 0]
    assert g["status"][6] == o["status"][6]
    assert np.all(g["accepted"][:5] == -1) and np.all(g["tokens"][:5] == -1)
    # at T = 1 a top-p cut within 1e-6 of 0.95 is a few-percent event per
    # distribution; a row is excluded only when it decides the outcome
    print(compare(g, o, "status", max_near=0.13))


def test_tiny_vocab_distribution_and_parity():
    # V = 8, 2*10^5 rounds as rows: GPU decisions match the oracle's and every
    # emitted position follows the filtered target distribution
    rounds, K, V, T, tp, mp = 200_000, 3, 8, 0.9, 0.95, 0.05
    rng = np.random.default_rng(12)
    z1 = rng.normal(0, 1.5, (K + 1, V)).astype(np.float32)
    d1 = (z1[:K] + rng.normal(0, 1.0, (K, V))).astype(np.float32)
    qf = [S.filtered(d1[i], T, tp, float(np.float32(mp)))[0] for i in range(K)]
    x = np.stack([rng.choice(V, size=rounds, p=qf[i] / qf[i].sum()) for i in range(K)], 1).astype(np.int32)
    z = np.ascontiguousarray(np.broadcast_to(z1, (rounds, K + 1, V)))
    d = np.ascontiguousarray(np.broadcast_to(d1, (rounds, K, V)))
    dev = torch.device("cuda:0")
    res = sv.accept_sampled(torch.from_numpy(z).to(dev), torch.from_numpy(d).to(dev),
                            torch.from_numpy(x).to(dev), temperature=T, top_p=tp, min_p=mp,
                            seed=21, offset=0)
    torch.cuda.synchronize()
    tok, acc = res.tokens.cpu().numpy(), res.accepted.cpu().numpy()
    pv = []
    for j in range(K + 1):
        pj = S.filtered(z1[j], T, tp, float(np.float32(mp)))[0]
        t = tok[acc >= j, j]
        cnt = np.bincount(t, minlength=V)
        sup = pj > 0
        assert cnt[~sup].sum() == 0
        if sup.sum() > 1:
            pv.append(scipy.stats.chisquare(cnt[sup], pj[sup] * cnt.sum()).pvalue)
    assert min(pv) > 1e-4 / len(pv), pv
    # parity on the first 3000 rounds
    o = S.spec_accept_sampled(z[:3000], d[:3000], x[:3000], None, T, T, tp, mp, 21, 0)
    g = {"tokens": tok[:3000], "accepted": acc[:3000], "p_draft": res.p_draft[:3000].cpu().numpy(),
         "status": res.status[:3000].cpu().numpy()}
    compare(g, o, "tiny")


def test_deterministic_and_row_shard_invariant():
    z, d, x, L = make_inputs(12, 4, 12000, std=3.0, noise=1.0, T=0.6, top_p=0.95, min_p=0.05,
                             seed=15, bf16=True, ragged=True)
    dev = torch.device("cuda:0")
    zt = torch.from_numpy(z).to(torch.bfloat16).to(dev)
    dtt = torch.from_numpy(d).to(torch.bfloat16).to(dev)
    xt, Lt = torch.from_numpy(x).to(dev), torch.from_numpy(L).to(dev)
    kw = dict(temperature=0.6, top_p=0.95, min_p=0.05, seed=3, offset=2)
    a1 = sv.accept_sampled(zt, dtt, xt, Lt, **kw)
    a2 = sv.accept_sampled(zt, dtt, xt, Lt, **kw)
    h = 5
    lo = sv.accept_sampled(zt[:h].contiguous(), dtt[:h].contiguous(), xt[:h].contiguous(),
                           Lt[:h].contiguous(), row_base=0, **kw)
    hi = sv.accept_sampled(zt[h:].contiguous(), dtt[h:].contiguous(), xt[h:].contiguous(),
                           Lt[h:].contiguous(), row_base=h, **kw)
    torch.cuda.synchronize()
    for f in ("tokens", "accepted", "p_draft", "status"):
        u, v = getattr(a1, f), getattr(a2, f)
        assert torch.equal(u, v), f
        assert torch.equal(u, torch.cat([getattr(lo, f), getattr(hi, f)])), f


@pytest.mark.parametrize("V,bf16,T,top_p,min_p", [
    (128256, True, 1.0, 0.5, 0.0),
    (128256, True, 0.6, 0.95, 0.05),
    (128256, True, 1.0, 0.95, 0.0),
    (20000, False, 1.0, 0.9, 0.0),
])
def test_large_crossing_bin_exact(V, bf16, T, top_p, min_p):
    # near-flat logits (std 0.02): the top-p cut falls in a bin of u that
    # holds tens of thousands of entries, more than the statistics kernel
    # collects in LDS, so each radix digit of the cut comes from a pass over
    # the row.  bf16 makes ~1000 distinct values of ~100 entries each, so a
    # cut within 1e-6 of top_p (an excluded row) stays rare.  With min-p on,
    # every entry passes it and the one-pass collection overflows too.
    z, d, x, L = make_inputs(6, 2, V, std=0.02, noise=0.01, T=T, top_p=top_p, min_p=min_p,
                             seed=60 + V % 7, bf16=bf16)
    g, o = run(z, d, x, L, T=T, top_p=top_p, min_p=min_p, seed=13, offset=3, bf16=bf16,
               label=f"large crossing bin V={V}")
    st = compare(g, o, ("large crossing bin", V, top_p, min_p), max_near=0.34)
    print(st)
    assert st["rows"] - st["near"] >= 4


def test_cut_in_the_unbinned_tail():
    # one dominant token and the rest 25 logit units below it (weights
    # < 2^-32 of the max, past the binned range): a top-p of 1 - 2^-22 puts
    # the cut among the tail entries.  Their masses are far inside the 1e-6
    # window, so the oracle marks every such cut near; the outputs must still
    # be valid draws from the kept set.
    B, K, V, T = 4, 2, 50000, 1.0
    rng = np.random.default_rng(71)
    z = np.full((B, K + 1, V), -25.0) + rng.normal(0, 0.5, (B, K + 1, V))
    z[:, :, 17] = 0.0
    z = z.astype(np.float32)
    d = z[:, :K].copy()
    x = np.full((B, K), 17, np.int32)
    tp = float(np.float32(1.0 - 2.0 ** -22))
    g, o = run(z, d, x, np.full(B, K, np.int32), T=T, top_p=tp, min_p=0.0, seed=2, offset=0,
               label="cut in the tail")
    assert np.all(g["status"] == 0) and np.all(g["accepted"] == K)
    assert np.all((g["tokens"] >= 0) & (g["tokens"] < V))
    ok = ~o["near"]
    assert np.array_equal(g["tokens"][ok], o["tokens"][ok])
