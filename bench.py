#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verification step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the verify linear layer on the lm-head (hidden [B(K+1), 4096] bf16 x W
[4096, 151936] bf16 -> fp32 logits) followed by the accept/reject pass over
those logits (B = 32 rows, K = 5 drafts, T = 0.6).  The headline value is
verified positions per second (B(K+1) per step).  The draft side (draft
probabilities from noisy target logits, draft tokens) is synthesised once,
untimed, on the GPU; every step draws a fresh Philox offset.

Also reported (``breakdown``): the accept/reject pass alone at B=64, K=7,
V=128256 bf16 with ragged draft lengths (rotating over 5 input sets, 1.8 GB,
so the 256 MB Infinity Cache cannot hold them), and the verify GEMM over the
M = B(1+D) sweep against W [4096, 14336] (rotating over 5 weight copies).

Also reported: verify attention (``spec_verify_attention``: the K+1 queries
of each sequence against its KV cache) at D = 0, 3, 7 on the pages' decode
example (8 sequences x 2048 tokens, 32 heads of 128) and on grouped-head
shapes (32 query / 8 KV heads), against the HBM roofline of the cache bytes;
the draft-depth controller (``spec_adapt``: telemetry and the
next depth per row, after each accept pass) at B=64 and B=4096, and the depth
planner (``spec_plan_depth``) fed with the GEMM sweep measured in the same
run, giving the best draft depth per batch size.

Roofline: the dominant kernel of the step is the lm-head GEMM; its achieved
bandwidth is its algorithmic bytes (2KN + 2MK + 4MN) over its average launch
duration, timed with HIP events on the stream it runs on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
# HBM bytes per call from FETCH_SIZE/WRITE_SIZE counter runs, calibrated on a
# plain copy; stamped with the digest of the kernel sources they describe
TRAFFIC_SUMMARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "traffic_lmhead_gemm_and_accept.md")
BF16_PEAK_TFLOPS = 2500.0
WARMUP_S = 0.5      # at least this long of untimed steps before the timed window
TEL_STEPS = 64      # untimed steps whose accept passes feed the acceptance telemetry


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-breakdown", action="store_true", help="time the step only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["step", "accept", "mid", "gemm", "adapt", "attn", "sampled"], default=None,
                    help="run one part only (for profiling)")
    return ap.parse_args()


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def _single_call_us(torch, fn, n=21):
    """Latency of one call: events around it and a synchronisation after
    each, so that no call overlaps another; the median over n calls."""
    ts = []
    for i in range(n):
        e0, e1 = _events(torch, 2)
        e0.record()
        fn(i)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    return sorted(ts)[n // 2]


def measured_peaks(torch, reps=10):
    """Practical peaks of this GPU, measured in the same process, as context
    beside the fractions of the published peaks: a device-to-device copy of
    1 GiB (bytes read plus bytes written per second) and the vendor library's
    bf16 product of two 8192 x 8192 matrices."""
    dev = torch.device("cuda:0")
    a = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    t0, t1 = _events(torch, 2)
    t0.record()
    for _ in range(reps):
        b.copy_(a)
    t1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * a.numel() * 2 * reps / (t0.elapsed_time(t1) * 1e-3) * 1e-9
    del a, b
    n = 8192
    X = torch.randn(n, n, device=dev).to(torch.bfloat16)
    W = torch.randn(n, n, device=dev).to(torch.bfloat16)
    Y = torch.matmul(X, W)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(reps):
        torch.matmul(X, W, out=Y)
    t1.record()
    torch.cuda.synchronize()
    tflops = 2 * n ** 3 * reps / (t0.elapsed_time(t1) * 1e-3) * 1e-12
    del X, W, Y
    return {"copy_GBs": round(copy_gbs, 1), "copy_frac_of_peak": round(copy_gbs / HBM_PEAK_GBS, 4),
            "matmul_bf16_TFLOPs": round(tflops, 1),
            "matmul_frac_of_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
            "how": "1 GiB device-to-device copy (read + written bytes); torch.matmul bf16 8192^3"}


def bench_step(torch, sv, workloads, steps, warmup):
    dev = torch.device("cuda:0")
    B, K, V, H = 32, 5, workloads.LMHEAD_N, workloads.HIDDEN
    M = B * (K + 1)
    hidden, W = workloads.linear_inputs(M, H, V, seed=5, device=dev)
    logits = torch.empty(M, V, dtype=torch.float32, device=dev)
    # the lm-head weight is static: it is stored once in the MFMA operand
    # order (spec_pack_weight), outside the timed steps, as a serving stack
    # would when it loads the model; the packing time is reported
    sv.pack_weight(W)
    torch.cuda.synchronize()
    t_pack = time.perf_counter()
    Wp = sv.pack_weight(W)
    torch.cuda.synchronize()
    pack_ms = (time.perf_counter() - t_pack) * 1e3
    ws_lin_n = sv.linear_packed_workspace_bytes(M, V, H)
    ws_lin = torch.empty(max(ws_lin_n, 1), dtype=torch.uint8, device=dev) if ws_lin_n else None
    sv.verify_linear_packed(hidden, Wp, V, out=logits, workspace=ws_lin)
    z3 = logits.view(B, K + 1, V)
    g = torch.Generator(device=dev)
    g.manual_seed(2005)
    q, x, L = workloads.draft_side_device(z3, K, 1.0, 0.6, g)
    ws_acc = sv.accept_workspace(B, K, V, dev)
    out = sv.AcceptResult(torch.empty(B, K + 1, dtype=torch.int32, device=dev),
                          torch.empty(B, dtype=torch.int32, device=dev),
                          torch.empty(B, K, dtype=torch.float32, device=dev),
                          torch.empty(B, dtype=torch.int32, device=dev))
    seed = 0x5EED

    def step(i, ev=None):
        if ev is not None:
            ev[0].record()
        sv.verify_linear_packed(hidden, Wp, V, out=logits, workspace=ws_lin)
        if ev is not None:
            ev[1].record()
        sv.accept(z3, q, x, L, temperature=0.6, seed=seed, offset=i, workspace=ws_acc, out=out)
        if ev is not None:
            ev[2].record()

    # warm-up: the requested steps, then more until WARMUP_S seconds of
    # steps have run, so that the timed window starts at steady clocks
    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < warmup or time.perf_counter() - t_w < WARMUP_S:
        step(n_warm)
        n_warm += 1
        if n_warm % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    base = n_warm
    # pass 1: whole-step throughput, nothing between launches
    t0, t1 = _events(torch, 2)
    t0.record()
    for i in range(steps):
        step(base + i)
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / steps
    # pass 2: per-step events (the dominant kernel's call, and the whole step)
    evs = [_events(torch, 3) for _ in range(steps)]
    for i in range(steps):
        step(base + steps + i, evs[i])
    torch.cuda.synchronize()
    gemm_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    # for comparison, the same product from W as stored (spec_verify_linear)
    ws_st_n = sv.linear_workspace_bytes(M, V, H)
    ws_st = torch.empty(max(ws_st_n, 1), dtype=torch.uint8, device=dev)
    for _ in range(3):
        sv.verify_linear(hidden, W, out=logits, workspace=ws_st)
    e0, e1 = _events(torch, 2)
    e0.record()
    for _ in range(steps):
        sv.verify_linear(hidden, W, out=logits, workspace=ws_st)
    e1.record()
    torch.cuda.synchronize()
    stored_ms = e0.elapsed_time(e1) / steps
    del ws_st
    step_ms = sorted(e[0].elapsed_time(e[2]) for e in evs)
    step_median_ms = step_ms[steps // 2]
    # pass 3: one step at a time, the GPU idle before each
    latency_ms = _single_call_us(torch, lambda i: step(base + 2 * steps + i)) * 1e-3
    # pass 4 (untimed): acceptance telemetry over TEL_STEPS further steps,
    # spec_adapt fed with each step's accepted lengths
    tel = sv.adapt_telemetry(dev)
    st_ad = sv.adapt_state(B, dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    resid_zero = torch.zeros((), dtype=torch.int64, device=dev)
    for i in range(TEL_STEPS):
        step(base + 3 * steps + 64 + i)
        sv.adapt(out.accepted, L, st_ad, tel, K=K, k_min=1, k_max=K, out=nxt)
        resid_zero += ((out.status & sv.ROW_RESID_ZERO) != 0).sum()
    torch.cuda.synchronize()
    acc = out.accepted.cpu()
    emitted = float((acc + 1).float().mean())
    gemm_bytes = 2 * H * V + 2 * M * H + 4 * M * V
    gemm_flops = 2 * M * H * V
    return dict(ms_per_step=ms_per_step, step_median_ms=step_median_ms, latency_ms=latency_ms,
                warmup_steps_run=n_warm, positions=M, gemm_ms=gemm_ms, gemm_bytes=gemm_bytes,
                stored_gemm_ms=stored_ms, pack_ms=pack_ms,
                gemm_flops=gemm_flops, mean_emitted=emitted,
                telemetry=_telemetry(sv, tel, K, int(resid_zero)),
                state=dict(hidden=hidden, W=W, logits=logits, q=q, x=x, L=L, B=B, K=K, V=V))


def _telemetry(sv, tel, K, resid_zero_rows):
    """Acceptance telemetry of the step's accept passes, from spec_adapt's
    counters: the acceptance rate, mean accepted length, per-position
    acceptance and the (draft length, accepted) histogram."""
    c = sv.telemetry_counters(tel)
    tested, accepted = c["tested_at"][:K], c["accepted_at"][:K]
    hist = c["hist"]
    al = {str(a): int(hist[:, a].sum()) for a in range(K + 1) if hist[:, a].sum()}
    return {"steps": int(c["calls"]), "rows": c["rows"], "invalid_rows": c["invalid_rows"],
            "acceptance_rate": round(c["accepted"] / max(c["tested"], 1), 4),
            "mean_accepted_drafts": round(c["accepted"] / max(c["rows"], 1), 4),
            "mean_emitted_per_pass": round(c["emitted"] / max(c["rows"], 1), 4),
            "per_position_acceptance": [round(int(a) / int(t), 4) if t else None
                                        for a, t in zip(accepted, tested)],
            "accepted_drafts_histogram": al,
            "zero_residual_rows": resid_zero_rows,
            "source": "spec_adapt counters over the accept passes of the telemetry steps"}


def bench_accept_large(torch, sv, workloads, reps=60, nsets=5):
    dev = torch.device("cuda:0")
    B, K, V = 64, 7, 128256
    sets = [workloads.large_accept_device(3000 + s, dev) for s in range(nsets)]
    ws = sv.accept_workspace(B, K, V, dev)
    outs = [sv.AcceptResult(torch.empty(B, K + 1, dtype=torch.int32, device=dev),
                            torch.empty(B, dtype=torch.int32, device=dev),
                            torch.empty(B, K, dtype=torch.float32, device=dev),
                            torch.empty(B, dtype=torch.int32, device=dev)) for _ in range(nsets)]
    positions, byts = [], []
    for s, (z, q, x, L) in enumerate(sets):
        sv.accept(z, q, x, L, temperature=0.8, seed=77, offset=s, workspace=ws, out=outs[s])
    torch.cuda.synchronize()
    for s, (z, q, x, L) in enumerate(sets):
        Lh = L.cpu().long()
        a = outs[s].accepted.cpu().long()
        rows = int((Lh + 1).sum())
        rej = int((a < Lh).sum())
        positions.append(rows)
        # every needed logits row once, one q row per rejecting row, the
        # token and q(x) gathers, and the outputs
        byts.append(rows * V * 2 + rej * V * 4 + int(Lh.sum()) * 8 + B * (K + 2) * 4)
    for r in range(5):
        for s, (z, q, x, L) in enumerate(sets):
            sv.accept(z, q, x, L, temperature=0.8, seed=77, offset=s, workspace=ws, out=outs[s])
    torch.cuda.synchronize()
    t0, t1 = _events(torch, 2)
    t0.record()
    for r in range(reps):
        for s, (z, q, x, L) in enumerate(sets):
            sv.accept(z, q, x, L, temperature=0.8, seed=77, offset=s, workspace=ws, out=outs[s])
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / (reps * nsets)

    def one(i):
        z, q, x, L = sets[i % nsets]
        sv.accept(z, q, x, L, temperature=0.8, seed=77, offset=i % nsets, workspace=ws,
                  out=outs[i % nsets])
    lat = _single_call_us(torch, one)
    pos = sum(positions) / nsets
    b = sum(byts) / nsets
    return dict(workload="spec_accept B=64 K=7 V=128256 bf16 T=0.8 ragged L~U{1..7}, 5 rotating sets",
                us_per_call=us, latency_us=lat, positions_per_call=pos, positions_per_s=pos / us * 1e6,
                algorithmic_bytes=b, achieved_GBs=b / us * 1e-3,
                frac_hbm=b / us * 1e-3 / HBM_PEAK_GBS)


def bench_accept_mid(torch, sv, workloads, reps=200):
    """The mid-size accept pass (B=8, K=4, V=32000 fp32, T=0.6, and its
    greedy variant with T=0 and argmax drafts): 40 positions and ~5 MB of
    logits per call, below the launch latency, so latency and positions/s
    are what it reports."""
    dev = torch.device("cuda:0")
    out = []
    for greedy in (False, True):
        inp = workloads.mid_accept(greedy=greedy)
        B, K1, V = inp.logits.shape
        K = K1 - 1
        z = inp.logits.to(dev)
        q = None if inp.draft_probs is None else torch.from_numpy(inp.draft_probs).to(dev)
        x = torch.from_numpy(inp.draft_tokens).to(dev)
        L = torch.from_numpy(inp.draft_lens).to(dev)
        ws = sv.accept_workspace(B, K, V, dev)
        res = sv.AcceptResult(torch.empty(B, K + 1, dtype=torch.int32, device=dev),
                              torch.empty(B, dtype=torch.int32, device=dev),
                              torch.empty(B, K, dtype=torch.float32, device=dev),
                              torch.empty(B, dtype=torch.int32, device=dev))
        T = inp.temperature

        def one(i):
            sv.accept(z, q, x, L, temperature=T, seed=inp.seed, offset=i, workspace=ws, out=res)
        for i in range(20):
            one(i)
        torch.cuda.synchronize()
        t0, t1 = _events(torch, 2)
        t0.record()
        for i in range(reps):
            one(i)
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / reps
        lat = _single_call_us(torch, one)
        pos = int((inp.draft_lens + 1).sum())
        out.append(dict(mode="greedy (T=0)" if greedy else "stochastic (T=0.6)", us_per_call=round(us, 2),
                        latency_us=round(lat, 2), positions_per_call=pos,
                        positions_per_s=round(pos / us * 1e6, 1),
                        logits_bytes=int(B * K1 * V * 4)))
    return dict(workload="spec_accept B=8 K=4 L=4 V=32000 fp32, z ~ N(0, 3^2), draft = z + N(0, 1)",
                bound="launch latency (~5 MB per call)", modes=out)


def bench_accept_sampled(torch, sv, workloads, reps=30, nsets=4):
    """Accept/reject with the draft as logits and the production sampler's
    filters (temperature 0.8 here as in the at-scale workload, top-p 0.95,
    min-p 0.05) at B=64, K=7, V=128256 bf16, ragged draft lengths."""
    dev = torch.device("cuda:0")
    B, K, V = 64, 7, 128256
    sets = [workloads.sampled_accept_device(4000 + s, dev) for s in range(nsets)]
    ws = sv.accept_sampled_workspace(B, K, V, dev)
    out = sv.AcceptResult(torch.empty(B, K + 1, dtype=torch.int32, device=dev),
                          torch.empty(B, dtype=torch.int32, device=dev),
                          torch.empty(B, K, dtype=torch.float32, device=dev),
                          torch.empty(B, dtype=torch.int32, device=dev))
    kw = dict(temperature=0.8, top_p=0.95, min_p=0.05, seed=77, workspace=ws, out=out)
    rows = []
    for s, (z, d, x, L) in enumerate(sets):
        sv.accept_sampled(z, d, x, L, offset=s, **kw)
        torch.cuda.synchronize()
        Lh = L.cpu().long()
        rows.append(int((Lh + 1).sum()) + int(Lh.sum()))
    t0, t1 = _events(torch, 2)
    t0.record()
    for r in range(reps):
        z, d, x, L = sets[r % nsets]
        sv.accept_sampled(z, d, x, L, offset=r, **kw)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / reps

    def one(i):
        z, d, x, L = sets[i % nsets]
        sv.accept_sampled(z, d, x, L, offset=i, **kw)
    lat = _single_call_us(torch, one)
    nrows = sum(rows) / nsets
    # every target row 0..L_b and draft row 0..L_b-1 read once, plus the
    # token gathers and outputs
    byts = nrows * V * 2 + B * (K + 2) * 4
    gbs = byts / us * 1e-3
    return dict(workload="spec_accept_sampled B=64 K=7 V=128256 bf16 target and draft logits, "
                         "T=0.8, top-p 0.95, min-p 0.05, ragged L~U{1..7}, draft = its top logit, "
                         f"{nsets} rotating sets",
                us_per_call=round(us, 2), latency_us=round(lat, 2), distributions_per_call=nrows,
                positions_per_s=round((nrows + B) / 2 / us * 1e6, 1),
                algorithmic_bytes=byts, achieved_GBs=round(gbs, 1),
                frac_hbm=round(gbs / HBM_PEAK_GBS, 4))


def bench_gemm_sweep(torch, sv, workloads, reps=40, ncopies=5):
    dev = torch.device("cuda:0")
    H, N = workloads.HIDDEN, workloads.FFN_N
    Ws = [workloads.linear_inputs(1, H, N, seed=900 + c, device=dev)[1] for c in range(ncopies)]
    res = []
    for M in workloads.sweep_ms():
        X = workloads.linear_inputs(M, H, 8, seed=M, device=dev)[0]
        Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        need = sv.linear_workspace_bytes(M, N, H)
        ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        for c in range(ncopies):
            sv.verify_linear(X, Ws[c], out=Y, workspace=ws)
        torch.cuda.synchronize()
        t0, t1 = _events(torch, 2)
        t0.record()
        for r in range(reps):
            for c in range(ncopies):
                sv.verify_linear(X, Ws[c], out=Y, workspace=ws)
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / (reps * ncopies)
        byts = 2 * H * N + 2 * M * H + 2 * M * N
        flops = 2 * M * H * N
        gbs = byts / us * 1e-3
        tfl = flops / us * 1e-6
        res.append(dict(M=M, us=round(us, 2), GBs=round(gbs, 1), TFLOPs=round(tfl, 1),
                        frac_hbm=round(gbs / HBM_PEAK_GBS, 3),
                        frac_mfma=round(tfl / BF16_PEAK_TFLOPS, 3)))
    return dict(workload="spec_verify_linear X[M,4096] x W[4096,14336] bf16 -> bf16, 5 rotating W copies",
                sweep=res)


def bench_attention(torch, sv, workloads, reps=30):
    """Verify attention per call at D = 0, 3, 7: the cache is read once per
    call whatever D is, so the time should stay flat in D while the rows
    grow (1+D)-fold."""
    import numpy as np
    dev = torch.device("cuda:0")
    cases = [("decode example, multi-head", 8, 32, 32, 2048, 1),
             ("grouped heads", 8, 32, 8, 8192, 1),
             ("grouped heads, 32 sequences", 32, 32, 8, 4096, 1),
             ("grouped heads, one long sequence", 1, 32, 8, 32768, 2)]
    res = []
    for label, B, H, Hkv, ctx_len, nsets in cases:
        row = {"case": label, "B": B, "H": H, "Hkv": Hkv, "ctx": ctx_len, "by_D": []}
        for D in (0, 3, 7):
            S = ctx_len + D + 1
            ctx = [ctx_len] * B
            sets = [workloads.attention_inputs(B, D, H, Hkv, ctx, S, seed=100 * D + k, device=dev)
                    for k in range(nsets)]
            out = torch.empty(B, D + 1, H, 128, dtype=torch.bfloat16, device=dev)
            need = sv.attention_workspace_bytes(B, D, H, Hkv, S)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            for k in range(nsets):
                q, kc, vc, ct, _ = sets[k]
                sv.verify_attention(q, kc, vc, ct, out=out, workspace=ws)
            torch.cuda.synchronize()
            t0, t1 = _events(torch, 2)
            t0.record()
            for r in range(reps):
                q, kc, vc, ct, _ = sets[r % nsets]
                sv.verify_attention(q, kc, vc, ct, out=out, workspace=ws)
            t1.record()
            torch.cuda.synchronize()
            us = t0.elapsed_time(t1) * 1e3 / reps
            kv = B * (ctx_len + D + 1) * Hkv * 128 * 2 * 2
            qo = 2 * B * (D + 1) * H * 128 * 2
            gbs = (kv + qo) / us * 1e-3
            row["by_D"].append(dict(D=D, rows_per_kv_head=(D + 1) * (H // Hkv), us=round(us, 2),
                                    bytes=kv + qo, GBs=round(gbs, 1),
                                    frac_hbm=round(gbs / HBM_PEAK_GBS, 3)))
            del sets, out, ws
        t = [r["us"] for r in row["by_D"]]
        row["time_D7_over_D0"] = round(t[2] / t[0], 3)
        res.append(row)
    return dict(workload="spec_verify_attention: q [B, D+1, H, 128] bf16 against k/v caches "
                         "[B, Hkv, ctx+D+1, 128] bf16, N(0,1), scale 1/sqrt(128), bf16 out",
                cases=res)


def bench_control(torch, sv, sweep, reps=200):
    """spec_adapt latency after an accept pass (the telemetry and the next
    depth per row), and the planner over the measured sweep."""
    dev = torch.device("cuda:0")
    K = 7
    out = {"adapt": []}
    for B in (64, 4096):
        g = torch.Generator(device=dev)
        g.manual_seed(B)
        L = torch.randint(1, K + 1, (B,), generator=g, device=dev, dtype=torch.int32)
        a = (torch.rand(B, generator=g, device=dev) * (L + 1).float()).floor().to(torch.int32)
        st, tel = sv.adapt_state(B, dev), sv.adapt_telemetry(dev)
        nxt = torch.empty(B, dtype=torch.int32, device=dev)
        kw = dict(K=K, k_min=1, k_max=K, window=8, policy=sv.ADAPT_SPEEDUP, draft_cost=0.05, out=nxt)
        for _ in range(10):
            sv.adapt(a, L, st, tel, **kw)
        torch.cuda.synchronize()
        # one launch is a few microseconds of GPU work, less than what the
        # Python binding takes to submit it: time a captured graph of `reps`
        # launches so that the host is out of the measurement
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for _ in range(reps):
                    sv.adapt(a, L, st, tel, **kw)
        torch.cuda.current_stream().wait_stream(side)
        graph.replay()
        torch.cuda.synchronize()
        t0, t1 = _events(torch, 2)
        t0.record()
        graph.replay()
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / reps
        # per row: a_b and L_b read, the 48-byte record read and written, the
        # next length written
        byts = B * (4 + 4 + 48 + 48 + 4)
        out["adapt"].append(dict(B=B, K=K, us_per_call=round(us, 2), bytes=byts,
                                 timing=f"graph of {reps} launches", bound="latency (one small launch)"))
    if not sweep:
        return out
    m = [r["M"] for r in sweep]
    t = [r["us"] for r in sweep]
    batches = [1, 2, 4, 8, 16, 32, 64, 128]
    plans = {}
    t0 = time.perf_counter()
    for alpha in (0.5, 0.7, 0.9):
        p = sv.plan_depth(m, t, batches, d_max=7, alpha=alpha, draft_cost=0.05)
        plans[f"alpha={alpha}"] = {str(b): {"D": int(p.best_depth[i]),
                                            "speedup": round(float(p.speedup[i, p.best_depth[i]]), 3)}
                                   for i, b in enumerate(batches)}
    host_us = (time.perf_counter() - t0) * 1e6 / 3
    out["plan"] = {"curve": "measured verify GEMM sweep above (one 4096x14336 layer)",
                   "draft_cost": 0.05, "d_max": 7, "best_depth_by_batch": plans,
                   "host_us_per_call": round(host_us, 1)}
    return out


def _host():
    """The host CPU model and its logical core count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count()}


def _timed(fn, budget_s):
    """Runs fn repeatedly for about budget_s (at least once): seconds per run."""
    n, t0 = 0, time.perf_counter()
    while n == 0 or time.perf_counter() - t0 < budget_s:
        fn()
        n += 1
    return (time.perf_counter() - t0) / n, n


def _cpu_rows(workloads, cores, budget_s=2.0):
    """The oracle, as it stands, on a bounded sample of each other measured
    path, scaled to that path's unit: the figures the GPU paths are set
    against in the breakdown."""
    import numpy as np

    import oracle
    from oracle import attention as A
    from oracle import control as C
    from oracle import sampled as S
    out = {}
    # accept/reject at scale (8 of the 64 rows; positions = sum(L_b + 1))
    inp = workloads.accept_inputs(8, 7, 128256, logit_std=3.0, draft_noise=1.5, temperature=0.8,
                                  seed=3, bf16=True, ragged=True)
    z = inp.logits_f32()
    pos = int((inp.draft_lens + 1).sum())
    sec, n = _timed(lambda: oracle.spec_accept(z, inp.draft_probs, inp.draft_tokens, inp.draft_lens,
                                                0.8, 77, 0, nthreads=cores), budget_s)
    out["accept_at_scale"] = dict(value=round(pos / sec, 1), unit="verified positions/s",
                                  sample=f"8 rows of B=64 K=7 V=128256, {n} run(s), {cores} threads")
    # the mid-size accept pass (all 8 rows, stochastic)
    mid = workloads.mid_accept()
    zm = mid.logits_f32()
    pm = int((mid.draft_lens + 1).sum())
    sec, n = _timed(lambda: oracle.spec_accept(zm, mid.draft_probs, mid.draft_tokens, mid.draft_lens,
                                                mid.temperature, mid.seed, 0, nthreads=cores), budget_s)
    out["accept_mid"] = dict(value=round(pm / sec, 1), unit="verified positions/s",
                             sample=f"all 8 rows of B=8 K=4 V=32000 fp32, {n} run(s), {cores} threads")
    # the sampler-filter path (2 rows)
    zs = z[:2]
    ds = (zs[:, :7] + np.random.default_rng(4).normal(0, 1.5, zs[:, :7].shape)).astype(np.float32)
    xs = ds.argmax(-1).astype(np.int32)
    Ls = inp.draft_lens[:2]
    sec, n = _timed(lambda: S.spec_accept_sampled(zs, ds, xs, Ls, 0.8, 0.8, 0.95, 0.05, 77, 0),
                    budget_s)
    out["accept_sampled_at_scale"] = dict(
        value=round(int((Ls + 1).sum()) / sec, 1), unit="verified positions/s",
        sample=f"2 rows of B=64 K=7 V=128256 with top-p 0.95, min-p 0.05, {n} run(s), 1 thread")
    # verify GEMM, M = 32 (fp64 matmul on an eighth of the columns, scaled)
    X = np.random.default_rng(5).normal(size=(32, 4096)).astype(np.float32)
    W = np.random.default_rng(6).normal(0, 0.02, size=(4096, 1792)).astype(np.float32)
    sec, n = _timed(lambda: oracle.verify_linear(X, W), budget_s)
    out["gemm_M32"] = dict(value=round(2 * 32 * 4096 * 1792 / sec * 1e-9, 2), unit="GFLOP/s",
                           sample=f"X[32,4096] x W[4096,1792] fp64, {n} run(s)")
    # verify attention: one query row against an 8192-token cache, scaled
    # to the 8 x 8192 grouped-head call at D = 7 (8 x 8 x 32 rows)
    rng = np.random.default_rng(7)
    q = rng.normal(size=(1, 8, 32, 128)).astype(np.float32)
    kc = rng.normal(size=(1, 8, 8200, 128)).astype(np.float32)
    vc = rng.normal(size=(1, 8, 8200, 128)).astype(np.float32)
    sec, n = _timed(lambda: A.verify_attention_row(q, kc, vc, 8192, 0, 7, 5, 128 ** -0.5), budget_s)
    out["verify_attention"] = dict(value=round(sec * 8 * 8 * 32 * 1e6, 1), unit="us per call",
                                   sample=f"one row of 8 x 8192 grouped-head D=7 scaled x2048, {n} run(s)")
    # depth controller, B = 4096
    rngc = np.random.default_rng(8)
    Lc = rngc.integers(1, 8, 4096)
    ac = np.floor(rngc.random(4096) * (Lc + 1)).astype(np.int64)
    stc, tel = C.new_state(4096), C.new_telemetry()
    sec, n = _timed(lambda: C.adapt(ac, Lc, 7, stc, tel, k_min=1, k_max=7, window=8, policy=1,
                                    draft_cost=0.05), budget_s)
    out["adapt_B4096"] = dict(value=round(sec * 1e6, 1), unit="us per call",
                              sample=f"B=4096 K=7, {n} run(s), 1 thread")
    return out


def cpu_baseline(torch, workloads, st, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample of the step: the fp64
    GEMM reference on a column slice of the lm-head (scaled to all columns)
    plus the fp64 accept/reject oracle on all 32 rows of the step."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    cores = max(1, min(cores, os.cpu_count() or 1))
    V, B, K = st["V"], st["B"], st["K"]
    ncols = V // 16
    Xh = st["hidden"].float().cpu().numpy()
    Wh = st["W"][:, :ncols].float().cpu().numpy()
    z = st["logits"].view(B, K + 1, V).cpu().numpy()
    q = st["q"].cpu().numpy()
    x = st["x"].cpu().numpy()
    L = st["L"].cpu().numpy()
    t_gemm, t_acc, n, near_rows = 0.0, 0.0, 0, 0
    t_start = time.perf_counter()
    while n == 0 or time.perf_counter() - t_start < budget_s:
        t0 = time.perf_counter()
        oracle.verify_linear(Xh, Wh)
        t1 = time.perf_counter()
        o = oracle.spec_accept(z, q, x, L, 0.6, 0x5EED, n, nthreads=cores)
        t2 = time.perf_counter()
        near_rows += int(np.sum((o["near_acc"] >= 0) | (o["near_smp"] > 0)))
        t_gemm += (t1 - t0) * (V / ncols)
        t_acc += t2 - t1
        n += 1
    per_step = (t_gemm + t_acc) / n
    rows = _cpu_rows(workloads, cores)
    return dict(value=round(B * (K + 1) / per_step, 2), unit="verified positions/s", paths=rows,
                cores=max(cores, blas_threads), kind="oracle",
                near_threshold_rows={"rows": near_rows, "of": n * B,
                                     "what": "rows of the oracle's runs on the step's logits whose "
                                             "acceptance test or draw lies within 1e-6 of its "
                                             "threshold"},
                sample=(f"{n} step(s): fp64 numpy GEMM on {ncols} of {V} lm-head columns scaled "
                        f"x{V / ncols:.0f} ({t_gemm / n:.2f} s/step) + fp64 C accept oracle on all "
                        f"{B} rows ({t_acc / n:.2f} s/step, {cores} OpenMP threads)"))


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the verification step would shard by rows, with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import speculative_decoding_verification_accept_amd as sv
    from speculative_decoding_verification_accept_amd import workloads

    if not os.path.exists(sv.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    sv.load_library()
    torch.cuda.set_device(0)

    if args.only == "accept":
        print(json.dumps(bench_accept_large(torch, sv, workloads)))
        return
    if args.only == "gemm":
        print(json.dumps(bench_gemm_sweep(torch, sv, workloads)))
        return
    if args.only == "mid":
        print(json.dumps(bench_accept_mid(torch, sv, workloads)))
        return
    if args.only == "sampled":
        print(json.dumps(bench_accept_sampled(torch, sv, workloads)))
        return
    if args.only == "attn":
        print(json.dumps(bench_attention(torch, sv, workloads)))
        return
    if args.only == "adapt":
        print(json.dumps(bench_control(torch, sv, [])))
        return

    import traffic
    counted = traffic.read_committed(TRAFFIC_SUMMARY)   # None once the kernels changed

    r = bench_step(torch, sv, workloads, args.steps, args.warmup)
    ms = r["ms_per_step"]
    value = r["positions"] / (ms * 1e-3)
    gemm_gbs = r["gemm_bytes"] / (r["gemm_ms"] * 1e-3) * 1e-9
    line = {
        "metric": "verified positions/s (spec_accept) & verify-GEMM TFLOPS; % HBM/MFMA roofline",
        "value": round(value, 1),
        "unit": "verified positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; hidden ~ N(0,1), W ~ N(0, 0.02^2), draft logits = target + N(0,1))",
        "config": {"workload": "fused verify step: lm-head GEMM hidden[192,4096] x W[4096,151936] "
                               "bf16 -> fp32 logits, then spec_accept B=32 K=5 V=151936 T=0.6",
                   "B": 32, "K": 5, "V": workloads.LMHEAD_N, "hidden": workloads.HIDDEN,
                   "M": r["positions"], "parallelism": "single GPU",
                   "lmhead_weight": "packed once in the MFMA operand order (spec_pack_weight), "
                                    "outside the timed steps"},
        "roofline": {"kernel": "spec_verify_linear_packed (lm-head, M=192)", "bound": "hbm",
                     "achieved": round(gemm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gemm_gbs / HBM_PEAK_GBS, 4),
                     "traffic": counted["lmhead_bytes"] if counted else None,
                     "avg_launch_us": round(r["gemm_ms"] * 1e3, 2),
                     "algorithmic_bytes": r["gemm_bytes"],
                     "tflops": round(r["gemm_flops"] / (r["gemm_ms"] * 1e-3) * 1e-12, 1),
                     "stored_weight_us": round(r["stored_gemm_ms"] * 1e3, 2),
                     "weight_pack_ms": round(r["pack_ms"], 3)},
        "mean_emitted_per_row": round(r["mean_emitted"], 3),
        "ms_per_step_median": round(r["step_median_ms"], 5),
        "single_step_latency_ms": round(r["latency_ms"], 4),
        "warmup_steps_run": r["warmup_steps_run"],
        "timing": (f"window: events around {args.steps} back-to-back steps after at least "
                   f"{args.warmup} steps and {WARMUP_S} s of untimed warm-up; median: per-step "
                   "events in a second pass; latency: one step with the GPU idle, median of 21"),
        "acceptance_telemetry": r["telemetry"],
        "host": _host(),
    }
    peaks = measured_peaks(torch)
    line["measured_peaks"] = peaks
    line["roofline"]["frac_of_measured_copy"] = round(gemm_gbs / peaks["copy_GBs"], 4)
    if not args.no_breakdown:
        acc = bench_accept_large(torch, sv, workloads)
        acc = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in acc.items()}
        acc["traffic_bytes"] = counted["accept_bytes"] if counted else None
        sweep = bench_gemm_sweep(torch, sv, workloads)
        line["breakdown"] = {"accept_at_scale": acc,
                             "accept_mid": bench_accept_mid(torch, sv, workloads),
                             "accept_sampled_at_scale": bench_accept_sampled(torch, sv, workloads),
                             "gemm_sweep": sweep,
                             "verify_attention": bench_attention(torch, sv, workloads),
                             "control": bench_control(torch, sv, sweep["sweep"])}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(torch, workloads, r["state"])
        line["acceptance_telemetry"]["near_threshold_rows"] = line["cpu_baseline"]["near_threshold_rows"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
