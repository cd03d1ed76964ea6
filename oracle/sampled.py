"""Oracle of the accept/reject pass with the production sampler's filters:
the draft is given as logits, and both the target's and the draft's
distributions pass through top-p and min-p before the acceptance rule.

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; the library's
product path never does.  It shares no code with the HIP implementation; the
Philox uniforms come from the C oracle (oracle.uniforms), written from the
generator's published definition.  fp64 throughout; a library sort, unique,
cumulative sum and search serve as steps.

Sources (cited by page title and section):
  [P2] "Decode is memory-bound: ~59 tok/s ceiling on an RTX 4090, and how
       speculative decoding beats it" (trefon.com), section "Two things that
       follow from the math": the production sampler settings (temperature
       0.6, top-p 0.95, min-p 0.05), the draft sampler matched to the
       target's, expected acceptance = the overlap sum of min(p, q);
       section "Speculative decoding": acceptance with probability
       min(1, p(x)/q(x)) makes the output exactly the target distribution.
  [P1] "Speculative decoding and early exit ..." (reactapp.top), section
       "Speculative decoding: draft first, then verify", listing
       speculative_decode: the draft distribution is the tempered softmax of
       the draft's logits; accept/reject, residual resample, bonus token.

Readings taken where the pages are silent:
  * A distribution is softmax(logits / T).  Top-p keeps token j iff the
    probability mass of the tokens with a strictly larger logit is below
    top_p (the smallest set of top tokens reaching top_p, ties at its edge
    kept together).  Min-p keeps j iff p_j >= min_p * max p.  Both are
    computed on the tempered, unfiltered distribution; a token is kept iff
    both keep it; the kept probabilities are renormalised.  top_p >= 1 and
    min_p <= 0 disable the respective filter.
  * The listing stops at the first rejection, so the target's distribution
    at position i is read only when every draft before it was accepted (the
    bonus position L only when all were): a non-finite target position makes
    the row invalid only if it is read, and p'_i(x_i) is reported for the
    tested positions only.  The drafted tokens are validated for all L
    drafts (range, finite draft logits, token in q''s kept set).
  * The target's filtered distribution p' and the draft's q' (with the
    draft's own temperature) replace p and q in the acceptance rule,
    residual and bonus draw of the unfiltered pass, with the same uniforms,
    inverse-CDF rule and fall-backs.  A draft token outside q''s kept set is
    a data error (ROW_ZERO_Q).
"""
from __future__ import annotations

import numpy as np

import oracle as _orc

ROW_NONFINITE = 1
ROW_BAD_TOKEN = 2
ROW_BAD_LEN = 4
ROW_ZERO_Q = 8
ROW_RESID_ZERO = 16
NEAR = 1e-6


def filtered(z, T: float, top_p: float, min_p: float):
    """(p' fp64 [V], kept bool [V], near: bool, nonfinite: bool) for one
    position's logits z.  `near` marks a filter decision within 1e-6 of its
    threshold (the mass above a kept/dropped boundary against top_p, or
    p_j / max p against min_p)."""
    z64 = np.asarray(z, dtype=np.float64)
    if not np.all(np.isfinite(z64) | (z64 == -np.inf)) or np.all(z64 == -np.inf):
        return None, None, False, True
    m = z64.max()
    e = np.exp((z64 - m) / T)          # p_j / max p
    p = e / e.sum()
    keep = np.ones(z64.shape[0], bool)
    near = False
    if top_p < 1.0:
        vals, inv = np.unique(z64, return_inverse=True)         # ascending values
        mass = np.bincount(inv, weights=p, minlength=vals.shape[0])
        above = np.cumsum(mass[::-1])[::-1] - mass             # mass of strictly larger values
        keep &= (above < top_p)[inv]
        near |= bool(np.any(np.abs(above - top_p) < NEAR))
    if min_p > 0.0:
        keep &= e >= min_p
        near |= bool(np.any(np.abs(e - min_p) < NEAR * min_p))
    pk = np.where(keep, p, 0.0)
    return pk / pk.sum(), keep, near, False


def near_tokens(z, T: float, top_p: float, min_p: float):
    """bool [V]: the tokens whose keep decision under the filters lies within
    1e-6 of its threshold (their value's mass-above against top_p, or p_j /
    max p against min_p); None for a non-finite position."""
    z64 = np.asarray(z, dtype=np.float64)
    if not np.all(np.isfinite(z64) | (z64 == -np.inf)) or np.all(z64 == -np.inf):
        return None
    m = z64.max()
    e = np.exp((z64 - m) / T)
    p = e / e.sum()
    near = np.zeros(z64.shape[0], bool)
    if top_p < 1.0:
        vals, inv = np.unique(z64, return_inverse=True)
        mass = np.bincount(inv, weights=p, minlength=vals.shape[0])
        above = np.cumsum(mass[::-1])[::-1] - mass
        near |= (np.abs(above - top_p) < NEAR)[inv]
    if min_p > 0.0:
        near |= np.abs(e - min_p) < NEAR * min_p
    return near


def _inv_cdf(w, u):
    """Smallest j whose inclusive prefix sum of w exceeds t = u * sum(w); the
    last positive j when rounding leaves none; `near` when t is within
    1e-6 * sum(w) of the chosen interval's ends."""
    c = np.cumsum(w)
    tot = c[-1]
    t = u * tot
    j = int(np.searchsorted(c, t, side="right"))
    pos = np.nonzero(w > 0)[0]
    if j >= w.shape[0] or w[j] <= 0:
        j = int(pos[-1])
    lo = c[j] - w[j]
    near = abs(t - lo) < NEAR * tot or abs(c[j] - t) < NEAR * tot
    return j, near


def spec_accept_sampled(target_logits, draft_logits, draft_tokens, draft_lens, T_target: float,
                        T_draft: float, top_p: float, min_p: float, seed: int, offset: int,
                        row_base: int = 0) -> dict:
    """target_logits [B, K+1, V], draft_logits [B, K, V] (fp32 values; bf16
    inputs widen exactly), draft_tokens [B, K], draft_lens [B] or None.
    Temperatures, top_p and min_p are rounded to fp32 as the GPU receives
    them.  Returns tokens [B, K+1] (-1 padded), accepted [B] (-1 invalid),
    p_draft [B, K] (p'_i(x_i) at the tested positions, -1 elsewhere), status
    [B], near [B] (a decision the row's outcome depends on lay within 1e-6
    of its threshold: a filter cut at a target position read or a draft
    position tested, the kept-set test of a draft token, an acceptance test
    or the draw)."""
    z = np.asarray(target_logits, dtype=np.float32)
    d = np.asarray(draft_logits, dtype=np.float32)
    B, K1, V = z.shape
    K = K1 - 1
    x = np.asarray(draft_tokens, dtype=np.int64).reshape(B, K)
    Ls = np.full(B, K) if draft_lens is None else np.asarray(draft_lens, dtype=np.int64)
    Tp, Tq = float(np.float32(T_target)), float(np.float32(T_draft))
    tp, mp = float(np.float32(top_p)), float(np.float32(min_p))
    out = dict(tokens=np.full((B, K1), -1, np.int32), accepted=np.full(B, -1, np.int32),
               p_draft=np.full((B, K), -1.0), status=np.zeros(B, np.int32),
               near=np.zeros(B, bool))
    for b in range(B):
        L = int(Ls[b])
        if L < 0 or L > K:
            out["status"][b] = ROW_BAD_LEN
            continue
        # the drafted tokens are validated for all L drafts: each draft
        # distribution q'_i, the token's range, and the token in q''s kept set
        st = 0
        qs, qnear = [], []
        for i in range(L):
            qf, _, nr, bad = filtered(d[b, i], Tq, tp, mp)
            st |= ROW_NONFINITE if bad else 0
            qs.append(qf)
            qnear.append(nr)
        ztok = []   # whether the kept-set test of x_i lies near a filter cut
        for i in range(L):
            if not 0 <= x[b, i] < V:
                st |= ROW_BAD_TOKEN
            elif qs[i] is not None:
                ztok.append(bool(near_tokens(d[b, i], Tq, tp, mp)[x[b, i]]))
                if not qs[i][x[b, i]] > 0.0:
                    st |= ROW_ZERO_Q
        if st:
            out["status"][b] = st
            out["near"][b] = any(ztok)
            continue
        # the target's distributions in the listing's order: position i only
        # when every draft before it was accepted, position L (the bonus) only
        # when all were; a non-finite position read this way makes the row
        # invalid, positions after the stop are never read
        gr = row_base + b
        a, nearrow, ps, bad = L, False, {}, False
        for i in range(L + 1):
            pf, _, nr, badp = filtered(z[b, i], Tp, tp, mp)
            if badp:
                bad = True
                break
            ps[i] = pf
            nearrow |= nr
            if i == L:
                break
            nearrow |= qnear[i]
            px, qx = pf[x[b, i]], qs[i][x[b, i]]
            out["p_draft"][b, i] = px
            acc = min(1.0, px / qx)
            ua, _ = _orc.uniforms(seed, offset, gr, i)
            nearrow |= abs(ua - acc) < NEAR
            if not ua < acc:
                a = i
                break
        # drafts past the stop matter only through their kept-set test
        nearrow |= any(ztok[a + 1:]) if not bad else any(ztok[i + 1:])
        if bad:
            out["p_draft"][b] = -1.0
            out["status"][b] = ROW_NONFINITE
            out["near"][b] = nearrow
            continue
        _, us = _orc.uniforms(seed, offset, gr, a)
        if a < L:
            w = np.maximum(ps[a] - qs[a], 0.0)
            if not w.sum() > 0.0:
                w = ps[a]
                st |= ROW_RESID_ZERO
        else:
            w = ps[L]
        tok, nr = _inv_cdf(w, us)
        nearrow |= nr
        out["tokens"][b, :a] = x[b, :a]
        out["tokens"][b, a] = tok
        out["accepted"][b] = a
        out["status"][b] = st
        out["near"][b] = nearrow
    return out


def acceptance_overlap(p, q) -> float:
    """Expected acceptance of one draft position: sum_j min(p_j, q_j)
    [P2 "Two things that follow from the math"]."""
    return float(np.minimum(p, q).sum())
