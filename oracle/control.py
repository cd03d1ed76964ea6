"""Oracle of the speculation controller: acceptance telemetry, the adaptive
draft-depth rule, and the depth planner over a measured verify-cost curve.

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; the library's
product path never does.  It shares no code with the HIP/C implementation.
Plain Python integers and IEEE doubles, rows and candidates visited in index
order, every floating-point expression written out in the order stated below
(Python never fuses a multiply into an add).

Sources (cited by page title and section):
  [P1] "Speculative decoding and early exit: accelerated autoregressive
       decoding" (reactapp.top), section "Production perspective" (ship the
       acceptance rate and the mean accepted length as metrics) and the
       operational checklist (record acceptance histograms).
  [P2] "Decode is memory-bound: ~59 tok/s ceiling on an RTX 4090, and how
       speculative decoding beats it" (trefon.com), section "Speculative
       decoding" (expected tokens per pass (1 - a^(k+1)) / (1 - a) for
       independent per-draft acceptance a; speedup with a draft step costing
       c of a target pass: that over (k c + 1)), section "Two things that
       follow from the math" (the fork's adaptive mode caps the draft depth
       once the measured acceptance drops under 35%), and the closing rules
       (pick the depth from the measured acceptance and keep measuring).
  [P3] agentnet.co.il item on speculative decoding, section "How it works in
       practice" (the accepted length lies in [1, 1+D]), section "The
       formula behind the speedup" (speculation pays when the verify time of
       B(1+D) rows, relative to that of B rows, is below the accepted length;
       the best D depends on B and moves along a Pareto frontier of
       throughput against interactivity), section "GEMM-M grows, a small
       batch suffices" (M = B(1+D)).

Readings taken where the pages are silent:
  * The measured acceptance of a row is the per-draft acceptance rate over
    the acceptance tests that actually ran: a pass that accepted a of L
    drafts ran a + 1 tests when a < L (the last one failed) and a tests when
    a = L.  Drafts past the first rejection were never tested and count as
    neither.  This is the estimate of the independent per-draft probability
    of [P2]'s formula.
  * "Measured" is over the row's last W passes (W <= 16), so the estimate
    follows the text as it changes ("keep measuring").  Passes with no test
    (L = 0) carry no information and are not recorded.
  * The threshold rule: with the measured acceptance below the floor (0.35
    in the fork), the depth drops to k_min; otherwise, and before any
    measurement, it is k_max.
  * The speedup rule: the depth in [k_min, k_max] that maximises
    E(a, k) / (k c + 1) at the measured a, the lowest such depth on ties;
    k_max before any measurement.  E is summed as 1 + a + a^2 + ... + a^k.
  * The planner prices a verify pass of M rows with a measured curve T(M),
    linear between measured points, flat below the first point and extended
    with the last segment's slope above the last.  A draft step at batch B
    costs c T(B).  Speedup over plain decoding at the same B:
        S(B, D) = E(a, D) T(B) / (T(B(1+D)) + D c T(B)),
    which is [P2]'s formula when T is flat and [P3]'s "verify time ratio
    below the accepted length" test when c = 0.
"""
from __future__ import annotations

import numpy as np

RING = 16                 # passes a row's record holds
STATE_BYTES = 64          # per-row record
MAX_K = 32                # largest draft depth the controller tracks
TEL_WORDS = 1200          # uint64 words of the telemetry block

# telemetry word offsets
T_ROWS, T_INVALID, T_DRAFTED, T_TESTED, T_ACCEPTED, T_EMITTED, T_CALLS = range(7)
T_TESTED_AT = 8                            # [MAX_K]
T_ACCEPTED_AT = T_TESTED_AT + MAX_K        # [MAX_K]
T_DEPTH_HIST = T_ACCEPTED_AT + MAX_K       # [MAX_K + 1]
T_HIST = T_DEPTH_HIST + MAX_K + 1          # [(MAX_K + 1) * (MAX_K + 1)], index L * (MAX_K + 1) + a

POLICY_THRESHOLD = 0
POLICY_SPEEDUP = 1


def new_state(B: int) -> np.ndarray:
    """Zeroed per-row records: no history."""
    return np.zeros((B, STATE_BYTES), np.uint8)


def new_telemetry() -> np.ndarray:
    return np.zeros(TEL_WORDS, np.uint64)


def expected_tokens_sum(alpha: float, k: int) -> float:
    """E(a, k) = 1 + a + ... + a^k: the expected tokens a pass emits when each
    of k drafts is accepted independently with probability a, stopping at the
    first rejection [P2 "Speculative decoding"].  Summed term by term with
    the power built by repeated multiplication."""
    e, term = 1.0, 1.0
    for _ in range(k):
        term = term * alpha
        e = e + term
    return e


def tests_run(a: int, L: int) -> int:
    """Acceptance tests a pass ran: the drafts accepted, plus the one that
    failed when the pass stopped before its last draft."""
    return a + (1 if a < L else 0)


def _ring_get(rec):
    succ = [int(v) for v in rec[0:RING]]
    trials = [int(v) for v in rec[RING:2 * RING]]
    count = int(rec[32]) | int(rec[33]) << 8 | int(rec[34]) << 16 | int(rec[35]) << 24
    return succ, trials, count


def _put_u32(rec, off, v):
    v &= 0xFFFFFFFF
    for i in range(4):
        rec[off + i] = (v >> (8 * i)) & 0xFF


def window_sums(rec, window: int):
    """(S, N): accepted drafts and tests over the record's last
    min(window, recorded) passes."""
    succ, trials, count = _ring_get(rec)
    S = N = 0
    for j in range(min(window, count, RING)):
        slot = (count - 1 - j) % RING
        S += succ[slot]
        N += trials[slot]
    return S, N


def choose_depth(S: int, N: int, k_min: int, k_max: int, policy: int, accept_floor: float,
                 draft_cost: float) -> int:
    """Next draft depth from the measured acceptance S / N [P2 "Two things
    that follow from the math", closing rules]."""
    if N == 0:
        return k_max
    if policy == POLICY_THRESHOLD:
        return k_min if float(S) < accept_floor * float(N) else k_max
    alpha = float(S) / float(N)
    best_k, best = k_min, -1.0
    for k in range(k_min, k_max + 1):
        g = expected_tokens_sum(alpha, k) / (float(k) * draft_cost + 1.0)
        if g > best:
            best_k, best = k, g
    return best_k


def adapt(accepted, draft_lens, K: int, state, telemetry, *, k_min: int, k_max: int,
          window: int, policy: int = POLICY_THRESHOLD, accept_floor: float = 0.35,
          draft_cost: float = 0.0):
    """One controller step after a verify pass.

    accepted   [B] int: a_b from the accept/reject pass (-1: invalid row)
    draft_lens [B] int or None (every row verified K drafts)
    state      [B, 64] uint8 records; telemetry [1200] uint64 counters
    Returns (next_lens [B] int32, new state, new telemetry); the inputs are
    not modified.
    """
    accepted = np.asarray(accepted).astype(np.int64)
    B = accepted.shape[0]
    lens = None if draft_lens is None else np.asarray(draft_lens).astype(np.int64)
    st = np.array(state, dtype=np.uint8, copy=True).reshape(B, STATE_BYTES)
    tel = [int(v) for v in np.asarray(telemetry, dtype=np.uint64)]
    nxt = np.zeros(B, np.int32)
    tel[T_CALLS] += 1
    for b in range(B):
        rec = st[b]
        L = K if lens is None else int(lens[b])
        a = int(accepted[b])
        if 0 <= L <= K and 0 <= a <= L:
            tests = tests_run(a, L)
            tel[T_ROWS] += 1
            tel[T_DRAFTED] += L
            tel[T_TESTED] += tests
            tel[T_ACCEPTED] += a
            tel[T_EMITTED] += a + 1
            tel[T_HIST + L * (MAX_K + 1) + a] += 1
            for i in range(tests):
                tel[T_TESTED_AT + i] += 1
            for i in range(a):
                tel[T_ACCEPTED_AT + i] += 1
            if tests > 0:
                _succ, _trials, count = _ring_get(rec)
                slot = count % RING
                rec[slot] = a
                rec[RING + slot] = tests
                _put_u32(rec, 32, count + 1)
        else:
            tel[T_INVALID] += 1
        S, N = window_sums(rec, window)
        d = choose_depth(S, N, k_min, k_max, policy, accept_floor, draft_cost)
        _put_u32(rec, 36, d)
        nxt[b] = d
        tel[T_DEPTH_HIST + d] += 1
    return nxt, st, np.array([v & 0xFFFFFFFFFFFFFFFF for v in tel], dtype=np.uint64)


def telemetry_summary(tel) -> dict:
    """Derived metrics of a telemetry block [P1 "Production perspective"]:
    acceptance rate, mean accepted length (AL = a + 1), per-position rates."""
    t = [int(v) for v in tel]
    rows = t[T_ROWS]
    tested_at = t[T_TESTED_AT:T_TESTED_AT + MAX_K]
    acc_at = t[T_ACCEPTED_AT:T_ACCEPTED_AT + MAX_K]
    return {
        "rows": rows, "invalid_rows": t[T_INVALID], "calls": t[T_CALLS],
        "acceptance_rate": t[T_ACCEPTED] / t[T_TESTED] if t[T_TESTED] else float("nan"),
        "mean_accepted_length": t[T_EMITTED] / rows if rows else float("nan"),
        "draft_efficiency": t[T_ACCEPTED] / t[T_DRAFTED] if t[T_DRAFTED] else float("nan"),
        "position_rates": [acc_at[i] / tested_at[i] if tested_at[i] else float("nan")
                           for i in range(MAX_K)],
    }


# --- planner -----------------------------------------------------------------

def verify_time(M: int, m_pts, t_pts) -> float:
    """T(M) from measured points (M ascending): linear between points, flat
    below the first, the last segment's slope above the last."""
    n = len(m_pts)
    if n == 1 or M <= m_pts[0]:
        return float(t_pts[0])
    j = 1
    while j < n - 1 and M > m_pts[j]:
        j += 1
    m0, m1 = float(m_pts[j - 1]), float(m_pts[j])
    t0, t1 = float(t_pts[j - 1]), float(t_pts[j])
    return t0 + ((t1 - t0) * (float(M) - m0)) / (m1 - m0)


def verify_rows(B: int, D: int) -> int:
    """Rows of every linear layer when B sequences verify D drafts each: each
    sequence verifies its D drafts plus the position after them [P3 "GEMM-M
    grows, a small batch suffices"]."""
    return B * (1 + D)


def plan_depth(m_pts, t_pts, batches, d_max: int, alpha: float, draft_cost: float):
    """For each batch size B and depth D in [0, d_max] [P2 "Speculative
    decoding" speedup formula; P3 "The formula behind the speedup"]:
        den = T(B(1+D)) + (D c) T(B)        pass time, draft steps included
        speedup = (E(a, D) T(B)) / den
        tokens_per_s = (B E(a, D)) / den * 1e6    (T in microseconds)
    Returns (best_depth [nB], speedup [nB, d_max+1], tokens_per_s [nB, d_max+1],
    pareto [nB, d_max+1] bool): the best depth maximises the speedup (lowest
    on ties); a point is on the Pareto frontier when no other (B, D) point
    has both total tokens/s and per-sequence tokens/s at least as high and
    one of them higher."""
    nB = len(batches)
    sp = np.zeros((nB, d_max + 1))
    rate = np.zeros((nB, d_max + 1))
    user = np.zeros((nB, d_max + 1))
    best = np.zeros(nB, np.int32)
    for bi, B in enumerate(batches):
        tb = verify_time(int(B), m_pts, t_pts)
        top = -1.0
        for D in range(d_max + 1):
            e = expected_tokens_sum(alpha, D)
            den = verify_time(verify_rows(int(B), D), m_pts, t_pts) + (float(D) * draft_cost) * tb
            s = (e * tb) / den
            sp[bi, D] = s
            rate[bi, D] = (float(B) * e) / den * 1e6
            user[bi, D] = e / den * 1e6
            if s > top:
                top, best[bi] = s, D
    pareto = np.zeros((nB, d_max + 1), bool)
    pts = [(rate[i, d], user[i, d]) for i in range(nB) for d in range(d_max + 1)]
    for idx, (x, y) in enumerate(pts):
        dominated = False
        for jdx, (x2, y2) in enumerate(pts):
            if jdx != idx and x2 >= x and y2 >= y and (x2 > x or y2 > y):
                dominated = True
                break
        pareto[idx // (d_max + 1), idx % (d_max + 1)] = not dominated
    return best, sp, rate, pareto
