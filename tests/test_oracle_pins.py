"""Pins of the fp64 accept/reject oracle against what the pages and the
mathematics fix, independent of any other implementation.

Sources:
  * page "Decode is memory-bound: ~59 tok/s ceiling on an RTX 4090, and how
    speculative decoding beats it" (trefon.com), section "Speculative
    decoding": acceptance rule min(1, p(x)/q(x)), exactness of the output
    distribution, the expected-tokens formula and its alpha-by-k table;
    section "Two things that follow from the math": expected acceptance is
    the overlap sum of min(p, q), and a greedy draft is accepted with the
    target's probability of that token.
  * page "Speculative decoding and early exit ..." (reactapp.top), section
    "Speculative decoding: draft first, then verify": worked value 3.36 and
    the accept/reject listing.
  * agentnet.co.il item, section "How it works in practice": the accepted
    length lies in [1, 1+D].
"""
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

from speculative_decoding_verification_accept_amd import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


# --- closed form ------------------------------------------------------------

def test_expected_tokens_table(oracle_mod):
    rows = _read_rows("expected_tokens_table.txt")
    assert len(rows) == 6
    for r in rows:
        a = float(r[0])
        for k, printed in zip((1, 3, 5), r[1:]):
            e = float(oracle_mod.expected_tokens_per_pass(a, k))
            # printed to two decimals, rounding half up (0.5, k=3 is 1.875)
            assert abs(e - float(printed)) <= 0.005 + 1e-12, (a, k, e, printed)


def test_expected_tokens_worked_examples(oracle_mod):
    for a, k, printed, tol, _src in _read_rows("worked_examples.txt"):
        e = float(oracle_mod.expected_tokens_per_pass(float(a), int(k)))
        assert abs(e - float(printed)) <= float(tol) + 1e-12, (a, k, e, printed)
    assert oracle_mod.expected_tokens_per_pass(0.8, 4) == pytest.approx(3.3616, abs=1e-12)
    assert oracle_mod.expected_tokens_positional([0.8] * 4) == pytest.approx(3.3616, abs=1e-12)


# --- helpers ----------------------------------------------------------------

def _binary_construction(alpha, k, rounds):
    """V=2, q=(1,0), p=(alpha, 1-alpha): every draft is token 0 and is accepted
    with probability exactly alpha; the residual max(p-q, 0) = (0, 1-alpha)
    always yields token 1."""
    z = np.log(np.array([alpha, 1.0 - alpha])).astype(np.float32)
    logits = np.ascontiguousarray(np.broadcast_to(z, (rounds, k + 1, 2)))
    q = np.zeros((rounds, k, 2), np.float32)
    q[..., 0] = 1.0
    x = np.zeros((rounds, k), np.int32)
    return logits, q, x


def _emitted_after(tokens, accepted, j):
    """Token emitted at position j by rows that reached position j."""
    sel = accepted >= j
    return tokens[sel, j]


def _chi2_p(tokens, p, V):
    counts = np.bincount(tokens, minlength=V)
    exp = p * counts.sum()
    keep = exp > 0
    assert counts[~keep].sum() == 0, "token with zero target probability emitted"
    return scipy.stats.chisquare(counts[keep], exp[keep] * counts[keep].sum() / exp[keep].sum()).pvalue


def _overlap(p, q):
    return np.minimum(p, q).sum()


# --- Monte Carlo against the closed form -----------------------------------

@pytest.mark.parametrize("alpha,k", [(0.8, 4), (0.5, 3), (0.9, 5), (0.35, 1)])
def test_mean_emitted_matches_closed_form(oracle_mod, alpha, k):
    rounds = 1_000_000
    logits, q, x = _binary_construction(alpha, k, rounds)
    out = oracle_mod.spec_accept(logits, q, x, None, 1.0, seed=123 + k, offset=0, nthreads=8)
    emitted = out["accepted"] + 1
    e = oracle_mod.expected_tokens_per_pass(alpha, k)
    # exact variance of the truncated geometric: P(emitted = n) = a^(n-1)(1-a) for n<=k, a^k for n=k+1
    n = np.arange(1, k + 2)
    pn = np.array([alpha ** (i - 1) * (1 - alpha) for i in n[:-1]] + [alpha ** k])
    sd = np.sqrt((pn * (n - e) ** 2).sum())
    assert abs(emitted.mean() - e) < 4 * sd / np.sqrt(rounds), (emitted.mean(), e)
    # a rejected row always resamples token 1 (the only residual mass)
    rej = out["accepted"] < k
    assert np.all(out["tokens"][rej, out["accepted"][rej]] == 1)
    # accepted length lies in [1, 1+D]
    assert emitted.min() >= 1 and emitted.max() <= k + 1


def test_acceptance_is_overlap_and_positional_expectation(oracle_mod):
    inp = workloads.small_accept(rounds=40000, seed=1)
    z, q1 = inp.meta["z"], inp.meta["q"]
    out = oracle_mod.spec_accept(inp.logits_f32(), inp.draft_probs, inp.draft_tokens,
                                 inp.draft_lens, inp.temperature, inp.seed, 0, nthreads=8)
    K = inp.K
    acc = out["accepted"]
    alphas = []
    for i in range(K):
        p = scipy.special.softmax(z[i].astype(np.float64) / inp.temperature)
        alpha = _overlap(p, q1[i].astype(np.float64))
        alphas.append(alpha)
        reached = acc >= i
        n = reached.sum()
        k_acc = (acc[reached] > i).sum()
        zstat = (k_acc - n * alpha) / np.sqrt(n * alpha * (1 - alpha))
        assert abs(zstat) < 4.5, (i, k_acc / n, alpha)
    e = oracle_mod.expected_tokens_positional(alphas)
    emitted = acc + 1
    assert abs(emitted.mean() - e) < 4.5 * emitted.std() / np.sqrt(len(emitted))


def test_residual_mass_identity(oracle_mod):
    # at every rejection, 1 - S_r equals the overlap sum of min(p, q)
    inp = workloads.small_accept(rounds=300, seed=5)
    z, q1 = inp.meta["z"], inp.meta["q"]
    out = oracle_mod.spec_accept(inp.logits_f32(), inp.draft_probs, inp.draft_tokens,
                                 inp.draft_lens, inp.temperature, inp.seed, 0)
    rej = np.nonzero(out["accepted"] < inp.K)[0]
    assert len(rej) > 50
    for b in rej[:100]:
        i = out["accepted"][b]
        p = scipy.special.softmax(z[i].astype(np.float64) / inp.temperature)
        assert abs((1 - out["resid_mass"][b]) - _overlap(p, q1[i].astype(np.float64))) < 1e-6


# --- exactness of the output distribution (V = 8) --------------------------

def _tiny_run(oracle_mod, rounds, K=4, T=1.0, seed=11, lens=None):
    inp = workloads.replicated_inputs(rounds, K, 8, logit_std=2.0, draft_noise=0.5,
                                      temperature=T, seed=seed, lens=lens)
    out = oracle_mod.spec_accept(inp.logits_f32(), inp.draft_probs, inp.draft_tokens,
                                 inp.draft_lens, inp.temperature, inp.seed, 0, nthreads=8)
    ps = [scipy.special.softmax(inp.meta["z"][i].astype(np.float64) / T) for i in range(K + 1)]
    return inp, out, ps


def _distribution_pvalues(out, ps, K):
    pv = []
    for j in range(K + 1):
        toks = _emitted_after(out["tokens"], out["accepted"], j)
        pv.append(_chi2_p(toks, ps[j], 8))
    return pv


def test_output_distribution_equals_target(oracle_mod):
    K = 4
    inp, out, ps = _tiny_run(oracle_mod, 1_000_000, K=K)
    pv = _distribution_pvalues(out, ps, K)
    assert min(pv) > 1e-4 / len(pv), pv
    # total variation of the first emitted token against p_0
    c = np.bincount(out["tokens"][:, 0], minlength=8) / len(out["tokens"])
    assert 0.5 * np.abs(c - ps[0]).sum() < 3e-3


def test_zero_drafts_is_plain_categorical(oracle_mod):
    # L_b = 0: the pass reduces to one categorical draw from p_0
    inp, out, ps = _tiny_run(oracle_mod, 200_000, K=3, lens=0)
    assert np.all(out["accepted"] == 0)
    assert _chi2_p(out["tokens"][:, 0], ps[0], 8) > 1e-4
    assert np.all(out["tokens"][:, 1:] == -1)
    # the draw is the inverse CDF of p_0 under the row's sampling uniform:
    # compare against numpy's searchsorted on the cumulative sum
    e = np.exp((inp.meta["z"][0].astype(np.float64) - inp.meta["z"][0].max()) / 1.0)
    c = np.cumsum(e)
    mism = 0
    for b in range(2000):
        _, u = oracle_mod.uniforms(inp.seed, 0, b, 0)
        ref = int(np.searchsorted(c, u * c[-1], side="right"))
        if ref != out["tokens"][b, 0]:
            mism += 1
            assert out["near_smp"][b] == 1
    assert mism <= 2


MUTATIONS = {
    1: "residual resampled from p instead of max(p - q, 0)",
    2: "residual operands swapped: max(q - p, 0)",
    3: "acceptance ratio transposed: q/p",
    4: "bonus drawn at position L-1 instead of L",
    5: "categorical draw reuses the acceptance uniform",
    6: "temperature ignored",
    7: "no stop at the first rejection",
    8: "acceptance test at position 0 skipped",
}


@pytest.mark.parametrize("m", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(oracle_mod, m):
    """Each plausible mistake planted in the oracle fails at least one of the
    distribution / acceptance pins (T = 0.7 so the temperature matters)."""
    K, T, rounds = 3, 0.7, 300_000
    oracle_mod.set_mutation(m)
    try:
        inp, out, ps = _tiny_run(oracle_mod, rounds, K=K, T=T, seed=21)
    finally:
        oracle_mod.set_mutation(0)
    pv = _distribution_pvalues(out, ps, K)
    acc = out["accepted"]
    zs = []
    for i in range(K):
        alpha = _overlap(ps[i], inp.meta["q"][i].astype(np.float64))
        reached = acc >= i
        n = reached.sum()
        k_acc = (acc[reached] > i).sum()
        zs.append(abs(k_acc - n * alpha) / np.sqrt(n * alpha * (1 - alpha)))
    caught = min(pv) < 1e-8 or max(zs) > 8
    assert caught, (MUTATIONS[m], pv, zs)


def test_unmutated_passes_same_check(oracle_mod):
    K, T = 3, 0.7
    inp, out, ps = _tiny_run(oracle_mod, 300_000, K=K, T=T, seed=21)
    pv = _distribution_pvalues(out, ps, K)
    assert min(pv) > 1e-4 / len(pv)


# --- greedy limit -------------------------------------------------------------

def _greedy_brute(z, x, L):
    B, K1, V = z.shape
    K = K1 - 1
    toks = np.full((B, K + 1), -1, np.int32)
    acc = np.zeros(B, np.int32)
    for b in range(B):
        g = [int(np.argmax(z[b, i])) for i in range(K + 1)]  # first index among ties
        a = 0
        while a < L[b] and x[b, a] == g[a]:
            a += 1
        toks[b, :a] = x[b, :a]
        toks[b, a] = g[a]
        acc[b] = a
    return toks, acc


def test_greedy_is_longest_prefix_match(oracle_mod):
    rng = np.random.default_rng(4)
    B, K, V = 64, 5, 300
    # bf16-like coarse logits so that ties are common
    z = np.round(rng.normal(0, 3, size=(B, K + 1, V)) * 2) / 2
    z = z.astype(np.float32)
    g = z.argmax(-1)
    # drafts agree with the argmax for a random prefix, then differ
    x = g[:, :K].copy().astype(np.int32)
    cut = rng.integers(0, K + 1, size=B)
    for b in range(B):
        if cut[b] < K:
            x[b, cut[b]] = (x[b, cut[b]] + 1 + rng.integers(0, V - 1)) % V
    L = rng.integers(0, K + 1, size=B).astype(np.int32)
    out = oracle_mod.spec_accept(z, None, x, L, 0.0, seed=1, offset=0)
    toks, acc = _greedy_brute(z, x, L)
    assert np.array_equal(out["accepted"], acc)
    assert np.array_equal(out["tokens"], toks)
    assert np.all(out["status"] == 0)


def test_greedy_ties_take_lowest_index(oracle_mod):
    z = np.zeros((1, 2, 10), np.float32)
    z[0, 0, [3, 7]] = 5.0
    z[0, 1, [2, 9]] = 1.0
    out = oracle_mod.spec_accept(z, None, np.array([[7]], np.int32), None, 0.0, 0, 0)
    assert out["accepted"][0] == 0 and out["tokens"][0, 0] == 3
    out = oracle_mod.spec_accept(z, None, np.array([[3]], np.int32), None, 0.0, 0, 0)
    assert out["accepted"][0] == 1 and list(out["tokens"][0]) == [3, 2]


# --- special cases ------------------------------------------------------------

def test_draft_equal_to_target_accepts_everything(oracle_mod):
    rounds, K, V, T = 2000, 4, 1000, 0.9
    rng = np.random.default_rng(8)
    z = rng.normal(0, 2, size=(K + 1, V)).astype(np.float32)
    q1 = workloads.draft_probs_from_logits(z[:K], T)
    logits = np.ascontiguousarray(np.broadcast_to(z, (rounds, K + 1, V)))
    q = np.ascontiguousarray(np.broadcast_to(q1, (rounds, K, V)))
    x = np.stack([rng.choice(V, size=rounds, p=q1[i] / q1[i].sum(dtype=np.float64))
                  for i in range(K)], 1).astype(np.int32)
    out = oracle_mod.spec_accept(logits, q, x, None, T, seed=3, offset=0)
    full = out["accepted"] == K
    # any rejection must have come from a near-threshold acceptance test
    assert np.all(full | (out["near_acc"] >= 0))
    assert full.mean() > 0.99


def test_one_hot_draft_accepts_with_target_probability(oracle_mod):
    # a greedy drafter puts all mass on one token: acceptance = p(that token)
    rounds, V, T = 200_000, 8, 0.6
    rng = np.random.default_rng(9)
    z = rng.normal(0, 2, size=(2, V)).astype(np.float32)
    xtok = int(np.argmax(z[0] + rng.normal(0, 1, V)))
    q1 = np.zeros((1, V), np.float32)
    q1[0, xtok] = 1.0
    logits = np.ascontiguousarray(np.broadcast_to(z, (rounds, 2, V)))
    q = np.ascontiguousarray(np.broadcast_to(q1, (rounds, 1, V)))
    x = np.full((rounds, 1), xtok, np.int32)
    out = oracle_mod.spec_accept(logits, q, x, None, T, seed=5, offset=0, nthreads=8)
    p = scipy.special.softmax(z[0].astype(np.float64) / np.float64(np.float32(T)))
    rate = (out["accepted"] == 1).mean()
    assert abs(rate - p[xtok]) < 4.5 * np.sqrt(p[xtok] * (1 - p[xtok]) / rounds)


def test_single_token_vocabulary(oracle_mod):
    B, K = 50, 3
    z = np.random.default_rng(1).normal(size=(B, K + 1, 1)).astype(np.float32)
    q = np.ones((B, K, 1), np.float32)
    x = np.zeros((B, K), np.int32)
    out = oracle_mod.spec_accept(z, q, x, None, 1.0, seed=1, offset=0)
    assert np.all(out["accepted"] == K) and np.all(out["tokens"] == 0)
    out = oracle_mod.spec_accept(z, None, x, None, 0.0, seed=1, offset=0)
    assert np.all(out["accepted"] == K) and np.all(out["tokens"] == 0)


def test_reproducible_and_row_shard_invariant(oracle_mod):
    inp = workloads.accept_inputs(16, 4, 500, logit_std=3.0, draft_noise=1.0,
                                  temperature=0.6, seed=12, ragged=True)
    z = inp.logits_f32()
    args = (inp.draft_probs, inp.draft_tokens, inp.draft_lens, inp.temperature, inp.seed, 77)
    full = oracle_mod.spec_accept(z, *args)
    again = oracle_mod.spec_accept(z, *args)
    for k in full:
        assert np.array_equal(full[k], again[k])
    h = 7
    lo = oracle_mod.spec_accept(z[:h], inp.draft_probs[:h], inp.draft_tokens[:h],
                                inp.draft_lens[:h], inp.temperature, inp.seed, 77, row_base=0)
    hi = oracle_mod.spec_accept(z[h:], inp.draft_probs[h:], inp.draft_tokens[h:],
                                inp.draft_lens[h:], inp.temperature, inp.seed, 77, row_base=h)
    for k in ("tokens", "accepted", "p_draft", "status"):
        assert np.array_equal(full[k], np.concatenate([lo[k], hi[k]]))
    # a different offset gives a different draw stream
    other = oracle_mod.spec_accept(z, *args[:-1], 78)
    assert not np.array_equal(full["tokens"], other["tokens"])


def test_accepted_length_bounds_ragged(oracle_mod):
    inp = workloads.accept_inputs(40, 7, 2000, logit_std=3.0, draft_noise=1.5,
                                  temperature=0.8, seed=13, ragged=True, bf16=True)
    out = oracle_mod.spec_accept(inp.logits_f32(), inp.draft_probs, inp.draft_tokens,
                                 inp.draft_lens, inp.temperature, inp.seed, 0)
    L = inp.draft_lens
    a = out["accepted"]
    assert np.all((a >= 0) & (a <= L))
    for b in range(inp.B):
        assert np.array_equal(out["tokens"][b, :a[b]], inp.draft_tokens[b, :a[b]])
        assert 0 <= out["tokens"][b, a[b]] < inp.V
        assert np.all(out["tokens"][b, a[b] + 1:] == -1)
        # p_draft holds p_i(x_i) at the tested positions i <= a_b (i < L_b)
        # and -1 after: the listing stops at the first rejection
        t = min(a[b] + 1, L[b])
        assert np.all(out["p_draft"][b, t:] == -1)
        assert np.all((out["p_draft"][b, :t] >= 0) & (out["p_draft"][b, :t] <= 1))


def test_p_draft_matches_textbook_softmax(oracle_mod):
    inp = workloads.accept_inputs(4, 3, 3000, logit_std=3.0, draft_noise=1.0,
                                  temperature=0.6, seed=14)
    z = inp.logits_f32()
    out = oracle_mod.spec_accept(z, inp.draft_probs, inp.draft_tokens, None,
                                 inp.temperature, inp.seed, 0)
    T = np.float64(np.float32(inp.temperature))
    for b in range(inp.B):
        tested = min(out["accepted"][b] + 1, inp.K)
        assert tested >= 1
        for i in range(tested):
            p = scipy.special.softmax(z[b, i].astype(np.float64) / T)
            assert out["p_draft"][b, i] == pytest.approx(p[inp.draft_tokens[b, i]], rel=1e-12)


# --- data errors --------------------------------------------------------------

def _base(B=3, K=2, V=16):
    rng = np.random.default_rng(0)
    z = rng.normal(size=(B, K + 1, V)).astype(np.float32)
    q = workloads.draft_probs_from_logits(z[:, :K], 1.0)
    x = np.zeros((B, K), np.int32)
    for b in range(B):
        for i in range(K):
            x[b, i] = int(np.argmax(q[b, i]))
    return z, q, x


def test_status_bits(oracle_mod):
    O = oracle_mod
    z, q, x = _base()
    z[0, 1, 5] = np.nan
    z[1, 2, 3] = np.inf
    z[2, 0, :] = -np.inf
    out = O.spec_accept(z, q, x, None, 1.0, 1, 0)
    assert list(out["status"]) == [O.ROW_NONFINITE] * 3
    assert np.all(out["accepted"] == -1) and np.all(out["tokens"] == -1)

    z, q, x = _base()
    z[0, 0, 4] = -np.inf  # a single -inf logit is a valid zero-probability token
    x[1, 1] = 16
    L = np.array([2, 2, 3], np.int32)
    out = O.spec_accept(z, q, x, L, 1.0, 1, 0)
    assert list(out["status"]) == [0, O.ROW_BAD_TOKEN, O.ROW_BAD_LEN]
    assert out["accepted"][0] >= 0 and out["accepted"][1] == -1

    z, q, x = _base()
    q[1, 0, x[1, 0]] = 0.0
    out = O.spec_accept(z, q, x, None, 1.0, 1, 0)
    assert list(out["status"]) == [0, O.ROW_ZERO_Q, 0]
    # greedy ignores q entirely
    out = O.spec_accept(z, None, x, None, 0.0, 1, 0)
    assert list(out["status"]) == [0, 0, 0]
    # a non-finite value past L_b is not read
    z, q, x = _base()
    z[0, 2, 0] = np.nan
    out = O.spec_accept(z, q, x, np.array([1, 2, 2], np.int32), 1.0, 1, 0)
    assert list(out["status"]) == [0, 0, 0]


def test_positions_after_the_first_rejection_are_not_read(oracle_mod):
    """The listing stops at the first rejection: a non-finite logit after it
    is never read (the row is valid), while one at or before it makes the
    row invalid; p_i(x_i) is reported for the tested positions only."""
    O = oracle_mod
    z, q, x = _base(B=3, K=3, V=16)
    # position 0: the draft token has all of q's mass but almost none of p's,
    # so the test at position 0 rejects (u < ~e^-30 never happens)
    for b in range(3):
        z[b, 0, :] = 0.0
        z[b, 0, 7] = -30.0
        q[b, 0, :] = 0.0
        q[b, 0, 7] = 1.0
        x[b, 0] = 7
    z[0, 1, 3] = np.nan           # after the rejection: not read
    z[1, 3, 2] = np.inf           # after the rejection: not read
    z[2, 0, 5] = np.nan           # at the rejected position: read
    out = O.spec_accept(z, q, x, None, 1.0, 5, 0)
    assert list(out["status"]) == [0, 0, O.ROW_NONFINITE]
    assert list(out["accepted"]) == [0, 0, -1]
    assert np.all(out["p_draft"][:2, 0] < 1e-12) and np.all(out["p_draft"][:2, 1:] == -1)
    assert np.all(out["p_draft"][2] == -1)
    # greedy: the same after the first disagreement with the argmax
    xg = x.copy()
    for b in range(3):
        xg[b, 0] = 8                # not the argmax of position 0 (token 0 ties win)
    out = O.spec_accept(z, None, xg, None, 0.0, 5, 0)
    assert list(out["status"]) == [0, 0, O.ROW_NONFINITE]
    assert list(out["accepted"]) == [0, 0, -1]


def test_invalid_arguments(oracle_mod):
    z, q, x = _base()
    with pytest.raises(ValueError):
        oracle_mod.spec_accept(z, None, x, None, 0.5, 1, 0)  # stochastic needs q
    with pytest.raises(ValueError):
        oracle_mod.spec_accept(z, q, x, None, -1.0, 1, 0)
    with pytest.raises(ValueError):
        oracle_mod.spec_accept(z, q, x, None, float("nan"), 1, 0)


# --- verify linear reference --------------------------------------------------

def test_verify_linear_reference_exact_on_integers(oracle_mod):
    rng = np.random.default_rng(3)
    M, K, N = 9, 64, 40
    X = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    W = rng.integers(-8, 9, size=(K, N)).astype(np.float32)
    Y = oracle_mod.verify_linear(X, W)
    Xi = X.astype(np.int64).tolist()
    Wi = W.astype(np.int64).tolist()
    for m in range(M):
        for n in range(N):
            assert Y[m, n] == sum(Xi[m][k] * Wi[k][n] for k in range(K))
    rows = rng.integers(0, M, 30)
    cols = rng.integers(0, N, 30)
    assert np.array_equal(oracle_mod.verify_linear_entries(X, W, rows, cols), Y[rows, cols])
