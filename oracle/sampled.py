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


def _filter_parts(z, T: float, top_p: float, min_p: float):
    """The pieces of one position's filtered distribution: (p fp64 [V], the
    top-p keep test [V], the min-p keep test [V], the ambiguous decisions),
    or None for a non-finite position.  An ambiguous decision is one value's
    keep test (criterion 0: top-p, its mass-above against top_p; 1: min-p,
    p_j / max p against min_p) that lies within 1e-6 of its threshold, with
    the mask of the tokens holding that value."""
    z64 = np.asarray(z, dtype=np.float64)
    if not np.all(np.isfinite(z64) | (z64 == -np.inf)) or np.all(z64 == -np.inf):
        return None
    m = z64.max()
    e = np.exp((z64 - m) / T)
    p = e / e.sum()
    top = np.ones(z64.shape[0], bool)
    mn = np.ones(z64.shape[0], bool)
    amb = []
    if top_p < 1.0:
        vals, inv = np.unique(z64, return_inverse=True)
        mass = np.bincount(inv, weights=p, minlength=vals.shape[0])
        above = np.cumsum(mass[::-1])[::-1] - mass
        top = (above < top_p)[inv]
        for k in np.nonzero(np.abs(above - top_p) < NEAR)[0]:
            amb.append((0, inv == k))
    if min_p > 0.0:
        mn = e >= min_p
        for v in np.unique(z64[np.abs(e - min_p) < NEAR * min_p]):
            amb.append((1, z64 == v))
    return p, top, mn, amb


def _renorm(parts, flips=()):
    """p' of a position with the ambiguous decisions `flips` (indices into
    its ambiguous list) taken the other way; None if nothing stays kept.
    With no flips this is filtered()'s p', the same operations."""
    p, top, mn, amb = parts
    if flips:
        top, mn = top.copy(), mn.copy()
        for k in flips:
            crit, mask = amb[k]
            if crit == 0:
                top[mask] = ~top[mask]
            else:
                mn[mask] = ~mn[mask]
    keep = top & mn
    pk = np.where(keep, p, 0.0)
    tot = pk.sum()
    return pk / tot if tot > 0.0 else None


def _row_outcome(L, K, V, xb, qd, pd, seed, offset, gr):
    """One row of the pass given q'_i (i < L) and p'_i (i <= L) (None: not
    finite).  Returns (status, a_b, tokens tuple, p_draft [K], near), near
    when the acceptance test or the draw lies within 1e-6 of its threshold;
    a_b = -1 and tokens None for an invalid row."""
    # the drafted tokens are validated for all L drafts: each draft
    # distribution q'_i, the token's range, and the token in q''s kept set
    st = 0
    for i in range(L):
        if qd[i] is None:
            st |= ROW_NONFINITE
        if not 0 <= xb[i] < V:
            st |= ROW_BAD_TOKEN
        elif qd[i] is not None and not qd[i][xb[i]] > 0.0:
            st |= ROW_ZERO_Q
    pdraft = np.full(K, -1.0)
    if st:
        return st, -1, None, pdraft, False
    # the target's distributions in the listing's order: position i only
    # when every draft before it was accepted, the bonus position L only when
    # all were; a non-finite position read this way makes the row invalid
    a, near = L, False
    for i in range(L + 1):
        if pd[i] is None:
            return ROW_NONFINITE, -1, None, np.full(K, -1.0), near
        if i == L:
            break
        px, qx = pd[i][xb[i]], qd[i][xb[i]]
        pdraft[i] = px
        acc = min(1.0, px / qx)
        ua, _ = _orc.uniforms(seed, offset, gr, i)
        near |= abs(ua - acc) < NEAR
        if not ua < acc:
            a = i
            break
    _, us = _orc.uniforms(seed, offset, gr, a)
    if a < L:
        w = np.maximum(pd[a] - qd[a], 0.0)
        if not w.sum() > 0.0:
            w = pd[a]
            st |= ROW_RESID_ZERO
    else:
        w = pd[L]
    tok, nr = _inv_cdf(w, us)
    return st, a, tuple(int(v) for v in xb[:a]) + (tok,), pdraft, near | nr


MAX_AMBIGUOUS = 4  # ambiguous filter decisions per row enumerated; more: the row is near


def spec_accept_sampled(target_logits, draft_logits, draft_tokens, draft_lens, T_target: float,
                        T_draft: float, top_p: float, min_p: float, seed: int, offset: int,
                        row_base: int = 0) -> dict:
    """target_logits [B, K+1, V], draft_logits [B, K, V] (fp32 values; bf16
    inputs widen exactly), draft_tokens [B, K], draft_lens [B] or None.
    Temperatures, top_p and min_p are rounded to fp32 as the GPU receives
    them.  Returns tokens [B, K+1] (-1 padded), accepted [B] (-1 invalid),
    p_draft [B, K] (p'_i(x_i) at the tested positions, -1 elsewhere), status
    [B], near [B] and p_draft_lo / p_draft_hi [B, K].

    near: the row's outcome (status, a_b, tokens) is not pinned to 1e-6 --
    its acceptance test or draw lies within 1e-6 of its threshold, or taking
    any of its ambiguous filter decisions (a keep test within 1e-6 of its
    threshold, in any of the row's distributions) the other way changes the
    outcome, or it has more than MAX_AMBIGUOUS of them.  Every combination
    of the ambiguous decisions is tried.  p_draft_lo / hi bound p'_i(x_i)
    over those combinations (equal to p_draft when none is ambiguous)."""
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
               near=np.zeros(B, bool), p_draft_lo=np.full((B, K), -1.0),
               p_draft_hi=np.full((B, K), -1.0))
    for b in range(B):
        L = int(Ls[b])
        if L < 0 or L > K:
            out["status"][b] = ROW_BAD_LEN
            continue
        gr = row_base + b
        qparts = [_filter_parts(d[b, i], Tq, tp, mp) for i in range(L)]
        pparts = [_filter_parts(z[b, i], Tp, tp, mp) for i in range(L + 1)]
        dists = qparts + pparts   # q'_0 .. q'_{L-1}, then p'_0 .. p'_L
        amb = [(k, j) for k, pa in enumerate(dists) if pa is not None for j in range(len(pa[3]))]
        nominal = [None if pa is None else _renorm(pa) for pa in dists]
        st, a, toks, pdraft, near = _row_outcome(L, K, V, x[b], nominal[:L], nominal[L:], seed, offset, gr)
        lo, hi = pdraft.copy(), pdraft.copy()
        if len(amb) > MAX_AMBIGUOUS:
            near = True
        else:
            for combo in range(1, 1 << len(amb)):
                flips = {}
                for bit, (k, j) in enumerate(amb):
                    if combo >> bit & 1:
                        flips.setdefault(k, []).append(j)
                alt = list(nominal)
                for k, js in flips.items():
                    alt[k] = _renorm(dists[k], tuple(js))
                if any(alt[k] is None for k in flips):
                    near = True
                    continue
                st2, a2, toks2, pd2, _ = _row_outcome(L, K, V, x[b], alt[:L], alt[L:], seed, offset, gr)
                if (st2, a2, toks2) != (st, a, toks):
                    near = True
                else:
                    t_ = pd2 >= 0
                    lo[t_] = np.minimum(lo[t_], pd2[t_])
                    hi[t_] = np.maximum(hi[t_], pd2[t_])
        out["status"][b] = st
        out["near"][b] = near
        out["p_draft"][b] = pdraft
        out["p_draft_lo"][b] = lo
        out["p_draft_hi"][b] = hi
        if toks is not None:
            out["accepted"][b] = a
            out["tokens"][b, :a + 1] = toks
    return out


def acceptance_overlap(p, q) -> float:
    """Expected acceptance of one draft position: sum_j min(p_j, q_j)
    [P2 "Two things that follow from the math"]."""
    return float(np.minimum(p, q).sum())
