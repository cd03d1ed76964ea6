"""Comparison of spec_accept's GPU outputs with the fp64 oracle's.

Decisions must agree exactly, except on rows where the oracle reports a draw
within 1e-6 of its threshold (an acceptance uniform within 1e-6 of
min(1, p/q), or a categorical draw within 1e-6 * total weight of a bracketing
prefix sum).  For such a row the outputs must still agree up to that draw;
the row is counted as excluded.  Probabilities p_i(x_i) must agree within
1e-5 relative.
"""
from __future__ import annotations

import numpy as np

P_RTOL = 1e-5


def compare(gpu: dict, orc: dict, K: int, max_excluded_frac: float = 0.01,
            label: str = "") -> dict:
    g_tok, o_tok = gpu["tokens"], orc["tokens"]
    g_acc, o_acc = gpu["accepted"], orc["accepted"]
    B = len(o_acc)
    same = np.all(g_tok == o_tok, axis=1) & (g_acc == o_acc)
    bad = []
    excluded = 0
    for b in np.nonzero(~same)[0]:
        na, ns = int(orc["near_acc"][b]), int(orc["near_smp"][b])
        if na >= 0:
            ok = g_acc[b] >= na and np.array_equal(g_tok[b, :na], o_tok[b, :na])
        elif ns:
            a = o_acc[b]
            ok = g_acc[b] == a and np.array_equal(g_tok[b, :a], o_tok[b, :a])
        else:
            ok = False
        if ok:
            excluded += 1
        else:
            bad.append(int(b))
    if bad:
        b = bad[0]
        raise AssertionError(
            f"{label}: {len(bad)} rows differ without a near-threshold draw; first row {b}: "
            f"gpu accepted={g_acc[b]} tokens={g_tok[b].tolist()} | oracle accepted={o_acc[b]} "
            f"tokens={o_tok[b].tolist()} status={orc['status'][b]} near=({orc['near_acc'][b]},"
            f"{orc['near_smp'][b]})")
    # status bits: identical on rows compared exactly
    st_ok = (gpu["status"] == orc["status"]) | ~same
    assert np.all(st_ok), f"{label}: status differs on rows {np.nonzero(~st_ok)[0][:10]}"
    # probabilities of the drafted tokens
    op = orc["p_draft"]
    gp = gpu["p_draft"].astype(np.float64)
    have = op >= 0
    assert np.array_equal(gp >= 0, have), f"{label}: p_draft coverage differs"
    if have.any():
        rel = np.abs(gp[have] - op[have]) / np.maximum(op[have], 1e-37)
        assert rel.max() <= P_RTOL, f"{label}: p_draft max rel err {rel.max():.3g}"
        p_rel = float(rel.max())
    else:
        p_rel = 0.0
    assert excluded <= max(2, max_excluded_frac * B), f"{label}: {excluded} excluded rows of {B}"
    near_rows = int(np.sum((orc["near_acc"] >= 0) | (orc["near_smp"] > 0)))
    return dict(rows=B, exact=int(same.sum()), excluded=excluded, near_rows=near_rows,
                p_draft_max_rel=p_rel)


def gpu_to_numpy(res) -> dict:
    return dict(tokens=res.tokens.cpu().numpy(), accepted=res.accepted.cpu().numpy(),
                p_draft=res.p_draft.cpu().numpy(), status=res.status.cpu().numpy())
