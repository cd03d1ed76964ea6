"""Pins of the controller oracle (oracle/control.py): acceptance telemetry,
the adaptive draft-depth rule and the depth planner, against what the pages
and the mathematics fix.

Sources:
  * page "Decode is memory-bound: ~59 tok/s ceiling on an RTX 4090, and how
    speculative decoding beats it" (trefon.com), section "Speculative
    decoding": E = (1 - a^(k+1)) / (1 - a), its table, and the speedup
    E / (k c + 1); section "Two things that follow from the math": the
    adaptive mode's 35% floor.
  * page "Speculative decoding and early exit ..." (reactapp.top), section
    "Production perspective" and the operational checklist: acceptance rate,
    mean accepted length, acceptance histograms.
  * agentnet.co.il item, sections "The formula behind the speedup" and
    "GEMM-M grows, a small batch suffices": speedup when the verify-time
    ratio of B(1+D) to B rows is below the accepted length; with D = 7 an
    eighth of the batch reaches the compute-bound regime.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import control as C

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                out.append(line.split())
    return out


def _traces():
    traces, cur = [], None
    for tok in _lines("adapt_trace.txt"):
        if tok[0] == "trace":
            cur = {"K": int(tok[1]), "W": int(tok[2]), "floor": float(tok[3]),
                   "kmin": int(tok[4]), "kmax": int(tok[5]), "passes": []}
            traces.append(cur)
        elif tok[0] in ("totals", "tested_at", "accepted_at", "depth_hist"):
            cur[tok[0]] = tok[1:]
        else:
            cur["passes"].append(tuple(int(v) for v in tok))
    return traces


def _run_trace(tr):
    st, tel = C.new_state(1), C.new_telemetry()
    got = []
    for L, a, _ in tr["passes"]:
        nxt, st, tel = C.adapt([a], [L], tr["K"], st, tel, k_min=tr["kmin"], k_max=tr["kmax"],
                               window=tr["W"], accept_floor=tr["floor"])
        got.append(int(nxt[0]))
    return got, tel


@pytest.mark.parametrize("ti", [0, 1])
def test_adapt_hand_worked_trace(ti):
    tr = _traces()[ti]
    got, tel = _run_trace(tr)
    assert got == [n for _, _, n in tr["passes"]]
    if "totals" in tr:
        rows, inval, drafted, tested, acc, emitted = (int(v) for v in tr["totals"])
        t = [int(v) for v in tel]
        assert (t[C.T_ROWS], t[C.T_INVALID], t[C.T_DRAFTED], t[C.T_TESTED], t[C.T_ACCEPTED],
                t[C.T_EMITTED]) == (rows, inval, drafted, tested, acc, emitted)
        ta = [int(v) for v in tr["tested_at"]]
        aa = [int(v) for v in tr["accepted_at"]]
        assert t[C.T_TESTED_AT:C.T_TESTED_AT + len(ta)] == ta
        assert t[C.T_ACCEPTED_AT:C.T_ACCEPTED_AT + len(aa)] == aa
        assert sum(t[C.T_TESTED_AT:C.T_TESTED_AT + C.MAX_K]) == tested
        for kv in tr["depth_hist"]:
            d, n = (int(v) for v in kv.split(":"))
            assert t[C.T_DEPTH_HIST + d] == n
        assert t[C.T_CALLS] == len(tr["passes"])


def test_threshold_rule_exact_fractions():
    # the floor compare in fp64 agrees with exact rational arithmetic at every
    # S <= N <= 400 with 35% (equality is "not below")
    floor = Fraction(35, 100)
    for N in range(1, 401):
        for S in range(N + 1):
            want = 1 if Fraction(S, N) < floor else 5
            assert C.choose_depth(S, N, 1, 5, C.POLICY_THRESHOLD, 0.35, 0.0) == want, (S, N)
    assert C.choose_depth(0, 0, 1, 5, C.POLICY_THRESHOLD, 0.35, 0.0) == 5


def test_expected_tokens_sum_matches_pages_table():
    rows = _lines("expected_tokens_table.txt")
    for r in rows:
        a = float(r[0])
        for k, printed in zip((1, 3, 5), r[1:]):
            assert abs(C.expected_tokens_sum(a, k) - float(printed)) <= 0.005 + 1e-12
    # the term-by-term sum equals the geometric closed form
    for a in np.linspace(0.0, 0.999, 37):
        for k in range(0, 33):
            closed = (1.0 - a ** (k + 1)) / (1.0 - a)
            assert abs(C.expected_tokens_sum(float(a), k) - closed) <= 1e-12 * closed
    assert C.expected_tokens_sum(1.0, 7) == 8.0


def test_speedup_rule_hand_worked():
    for a, c, kmin, kmax, best in _lines("speedup_depth.txt"):
        a, c = float(a), float(c)
        # a = S/N exactly for these alphas with N = 100
        S = int(round(a * 100))
        assert C.choose_depth(S, 100, int(kmin), int(kmax), C.POLICY_SPEEDUP, 0.35, c) == int(best)


def test_speedup_rule_argmax_brute_force():
    rng = np.random.default_rng(4)
    for _ in range(400):
        N = int(rng.integers(1, 200))
        S = int(rng.integers(0, N + 1))
        c = float(rng.choice([0.0, 0.02, 0.05, 0.1, 0.3, 1.0]))
        kmin = int(rng.integers(1, 4))
        kmax = int(rng.integers(kmin, 12))
        a = S / N
        vals = [((1 - a ** (k + 1)) / (1 - a) if a < 1 else k + 1.0) / (k * c + 1)
                for k in range(kmin, kmax + 1)]
        top = max(vals)
        got = C.choose_depth(S, N, kmin, kmax, C.POLICY_SPEEDUP, 0.35, c)
        # the choice is a maximiser (up to rounding) and no lower depth is
        # clearly better
        assert vals[got - kmin] >= top * (1 - 1e-12)
        assert all(v <= vals[got - kmin] * (1 + 1e-12) for v in vals[:got - kmin])


def _simulate(alphas, L, passes, B, seed, window=16):
    """Rows drafting L tokens, position i accepted with probability
    alphas[i], stopping at the first rejection (drawn on the CPU)."""
    rng = np.random.default_rng(seed)
    st, tel = C.new_state(B), C.new_telemetry()
    for _ in range(passes):
        u = rng.random((B, L))
        ok = u < np.asarray(alphas)[None, :L]
        a = np.where(ok.all(1), L, np.argmin(ok, axis=1))
        _, st, tel = C.adapt(a, np.full(B, L), L, st, tel, k_min=1, k_max=L, window=window)
    return st, tel


def test_acceptance_estimate_recovers_alpha():
    # the estimate is the per-draft probability of the pages' formula: with
    # i.i.d. acceptance a the rate over tests run converges to a (4 sigma)
    for alpha in (0.35, 0.6, 0.9):
        st, tel = _simulate([alpha] * 5, 5, passes=40, B=500, seed=int(alpha * 100))
        s = C.telemetry_summary(tel)
        n = int(tel[C.T_TESTED])
        sigma = math.sqrt(alpha * (1 - alpha) / n)
        assert abs(s["acceptance_rate"] - alpha) < 4 * sigma, (alpha, s["acceptance_rate"])
        # mean accepted length against the closed form E(a, L)
        e = C.expected_tokens_sum(alpha, 5)
        rows = int(tel[C.T_ROWS])
        assert abs(s["mean_accepted_length"] - e) < 4 * 1.6 / math.sqrt(rows)


def test_position_rates_and_positional_formula():
    import oracle
    alphas = [0.9, 0.7, 0.5, 0.8]
    st, tel = _simulate(alphas, 4, passes=30, B=700, seed=3)
    s = C.telemetry_summary(tel)
    t = [int(v) for v in tel]
    for i, a in enumerate(alphas):
        n = t[C.T_TESTED_AT + i]
        assert abs(s["position_rates"][i] - a) < 4 * math.sqrt(a * (1 - a) / n), i
    e = oracle.expected_tokens_positional(alphas)
    assert abs(s["mean_accepted_length"] - e) < 4 * 1.3 / math.sqrt(t[C.T_ROWS])
    # histogram invariants: counts add up to rows and emitted tokens
    hist = np.array(t[C.T_HIST:C.T_HIST + (C.MAX_K + 1) ** 2]).reshape(C.MAX_K + 1, C.MAX_K + 1)
    assert hist.sum() == t[C.T_ROWS]
    assert (hist * (np.arange(C.MAX_K + 1)[None, :] + 1)).sum() == t[C.T_EMITTED]
    assert hist[4].sum() == t[C.T_ROWS]            # every row drafted L = 4


def test_controller_tracks_acceptance_changes():
    # acceptance falls to 0.2 then recovers to 0.9: with a window of 8 passes
    # the threshold rule cuts the depth, then restores it.  At depth 1 a pass
    # runs one test, so the window holds Binomial(8, 0.2) successes and
    # P(S >= 3) ~ 0.2 of the rows measure >= 35% and go back up for a pass.
    B, L = 400, 5
    rng = np.random.default_rng(9)
    st, tel = C.new_state(B), C.new_telemetry()
    lens = np.full(B, L)
    frac_low = []
    for phase_alpha in (0.9, 0.2, 0.9):
        for _ in range(12):
            u = rng.random((B, L))
            ok = u < phase_alpha
            ok &= np.arange(L)[None, :] < lens[:, None]
            a = np.where(ok[:, :L].all(1), lens, np.argmin(ok, axis=1))
            a = np.minimum(a, lens)
            nxt, st, tel = C.adapt(a, lens, L, st, tel, k_min=1, k_max=L, window=8)
            lens = nxt.astype(np.int64)
        frac_low.append(float((lens == 1).mean()))
    assert frac_low[0] < 0.05 and frac_low[1] > 0.7 and frac_low[2] < 0.05, frac_low


def test_planted_trial_count_mistake_is_caught(monkeypatch):
    # counting every drafted token as a test (a / L) biases the estimate low
    monkeypatch.setattr(C, "tests_run", lambda a, L: L)
    st, tel = _simulate([0.6] * 5, 5, passes=40, B=500, seed=60)
    s = C.telemetry_summary(tel)
    sigma = math.sqrt(0.6 * 0.4 / int(tel[C.T_TESTED]))
    assert abs(s["acceptance_rate"] - 0.6) > 4 * sigma


# --- planner -----------------------------------------------------------------

def test_verify_time_interpolation():
    m, t = [1, 8, 64, 512], [20.0, 22.0, 30.0, 100.0]
    for mi, ti in zip(m, t):
        assert C.verify_time(mi, m, t) == ti
    assert C.verify_time(0, m, t) == 20.0
    assert C.verify_time(36, m, t) == pytest.approx(26.0, abs=1e-12)
    # above the last point: the last segment's slope (70 us per 448 rows)
    assert C.verify_time(960, m, t) == pytest.approx(170.0, abs=1e-9)
    assert C.verify_time(5, [4], [9.0]) == 9.0


def test_planner_flat_cost_is_the_pages_formula():
    m, t = [1, 4096], [50.0, 50.0]
    for alpha in (0.35, 0.5, 0.7, 0.9):
        for c in (0.0, 0.05, 0.2):
            best, sp, rate, _ = C.plan_depth(m, t, [1, 8, 64], 7, alpha, c)
            for D in range(8):
                want = ((1 - alpha ** (D + 1)) / (1 - alpha)) / (D * c + 1)
                assert np.allclose(sp[:, D], want, rtol=1e-12, atol=0)
            assert np.allclose(rate[1], 8 * rate[0], rtol=1e-12)


def test_planner_speedup_ratio_rule():
    # c = 0: speculation pays exactly when T(B(1+D)) / T(B) < E(a, D)
    m = [1, 4, 8, 32, 64, 128, 256, 512, 1024]
    t = [25.7, 26.0, 27.7, 28.3, 30.4, 33.8, 49.0, 85.0, 133.0]
    Bs = [1, 8, 32, 64, 128, 256]
    for alpha in (0.35, 0.6, 0.8):
        best, sp, rate, _ = C.plan_depth(m, t, Bs, 7, alpha, 0.0)
        for bi, B in enumerate(Bs):
            for D in range(8):
                ratio = C.verify_time(B * (1 + D), m, t) / C.verify_time(B, m, t)
                e = (1 - alpha ** (D + 1)) / (1 - alpha)
                if abs(ratio - e) > 1e-9:
                    assert (sp[bi, D] > 1.0) == (ratio < e), (alpha, B, D)
            assert sp[bi, best[bi]] == sp[bi].max()
    # compute-bound cost (T proportional to M) never pays for a < 1
    best, sp, _, _ = C.plan_depth([1, 2], [1.0, 2.0], [16, 64], 7, 0.8, 0.0)
    assert list(best) == [0, 0]


def test_planner_eighth_of_the_batch_at_depth_seven():
    # roofline-shaped cost: flat (memory-bound) up to M* rows, linear after.
    # With a = 1 and c = 0 the speedup stays exactly 1 + D while B(1+D) <= M*,
    # so the largest such batch at D = 7 is an eighth of that at D = 0's M*.
    Mstar = 512
    m, t = [1, Mstar, 2 * Mstar], [10.0, 10.0, 20.0]
    Bs = list(range(1, 2 * Mstar + 1))
    _, sp, _, _ = C.plan_depth(m, t, Bs, 7, 1.0, 0.0)
    last_mem = {D: max(B for bi, B in enumerate(Bs) if sp[bi, D] == 1 + D
                       and C.verify_time(B, m, t) == 10.0) for D in (1, 3, 7)}
    assert last_mem[7] == Mstar // 8 and last_mem[3] == Mstar // 4 and last_mem[1] == Mstar // 2


def test_planner_pareto_frontier_properties():
    m = [1, 4, 8, 32, 64, 128, 256, 512, 1024]
    t = [25.7, 26.0, 27.7, 28.3, 30.4, 33.8, 49.0, 85.0, 133.0]
    Bs = [1, 2, 4, 8, 16, 32, 64, 128]
    best, sp, rate, par = C.plan_depth(m, t, Bs, 7, 0.7, 0.05)
    E = np.array([C.expected_tokens_sum(0.7, D) for D in range(8)])
    user = rate / np.array(Bs, float)[:, None]
    pts = [(rate[i, d], user[i, d], par[i, d]) for i in range(len(Bs)) for d in range(8)]
    front = [(x, y) for x, y, p in pts if p]
    assert front
    for x, y, p in pts:
        dom = any(x2 >= x and y2 >= y and (x2 > x or y2 > y) for x2, y2, _ in pts)
        assert p == (not dom)
    # the best total rate and the best per-sequence rate are on the frontier
    i = int(np.argmax(rate))
    assert par.flat[i]
    j = int(np.argmax(user))
    assert par.flat[j]
    # along the frontier, more total throughput costs per-sequence rate
    front.sort()
    assert all(front[k][1] > front[k + 1][1] for k in range(len(front) - 1))
    assert np.allclose(user[:, 0] * 1e-6 * np.array([C.verify_time(B, m, t) for B in Bs]), E[0])


def test_planted_row_count_mistake_is_caught(monkeypatch):
    # pricing the pass at B*D rows (forgetting the position after the
    # drafts) breaks the eighth-of-the-batch pin
    monkeypatch.setattr(C, "verify_rows", lambda B, D: B * max(D, 1))
    with pytest.raises(AssertionError):
        test_planner_eighth_of_the_batch_at_depth_seven()
