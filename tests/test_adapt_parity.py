"""spec_adapt on the GPU against the controller oracle (oracle/control.py),
bit for bit: next draft lengths, the per-row records and every telemetry
counter, after every pass of multi-pass sequences.

Definition: page "Decode is memory-bound ..." (trefon.com), section "Two
things that follow from the math" (depth capped under 35% measured
acceptance) and the closing rules; page "Speculative decoding and early
exit ..." (reactapp.top), section "Production perspective" and the
operational checklist (acceptance rate, mean accepted length, histograms).
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verification_accept_amd as sv
from oracle import control as C
from speculative_decoding_verification_accept_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()
    oracle.set_mutation(0)
    sv.load_library()


def _passes(rng, B, K, n):
    """Random pass outcomes: L in [0, K], a in [0, L], with some invalid rows
    (a = -1 as the accept pass reports them, or a > L)."""
    for _ in range(n):
        L = rng.integers(0, K + 1, B).astype(np.int32)
        a = np.floor(rng.random(B) * (L + 1)).astype(np.int32)
        bad = rng.random(B) < 0.03
        a[bad] = -1
        worse = rng.random(B) < 0.01
        a[worse] = L[worse] + 1
        yield L, a


def _run(B, K, n, *, policy, window, k_min, k_max, floor=0.35, cost=0.0, seed=0, lens=True):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(seed)
    st_g, tel_g = sv.adapt_state(B, dev), sv.adapt_telemetry(dev)
    st_o, tel_o = C.new_state(B), C.new_telemetry()
    for p, (L, a) in enumerate(_passes(rng, B, K, n)):
        if not lens:
            L = np.full(B, K, np.int32)
            a = np.minimum(a, K)
        print(f"[spec_adapt] B={B} K={K} pass={p} policy={policy} W={window}", flush=True)
        nxt_g = sv.adapt(torch.from_numpy(a).to(dev), torch.from_numpy(L).to(dev) if lens else None,
                         st_g, tel_g, K=K, k_min=k_min, k_max=k_max, window=window, policy=policy,
                         accept_floor=floor, draft_cost=cost)
        torch.cuda.synchronize()
        nxt_o, st_o, tel_o = C.adapt(a, L if lens else None, K, st_o, tel_o, k_min=k_min,
                                     k_max=k_max, window=window, policy=policy,
                                     accept_floor=floor, draft_cost=cost)
        assert np.array_equal(nxt_g.cpu().numpy(), nxt_o), p
        assert np.array_equal(st_g.cpu().numpy(), st_o), p
        assert np.array_equal(tel_g.cpu().numpy().astype(np.uint64), tel_o), p
    return tel_o


@pytest.mark.parametrize("policy,window,cost", [(sv.ADAPT_THRESHOLD, 8, 0.0),
                                                (sv.ADAPT_THRESHOLD, 1, 0.0),
                                                (sv.ADAPT_SPEEDUP, 16, 0.05),
                                                (sv.ADAPT_SPEEDUP, 5, 0.3)])
def test_random_passes_bit_exact(policy, window, cost):
    tel = _run(1000, 7, 24, policy=policy, window=window, k_min=1, k_max=7, cost=cost, seed=window)
    assert int(tel[C.T_INVALID]) > 0 and int(tel[C.T_ROWS]) > 0


def test_max_depth_and_ragged_grid():
    # K = 32 (the controller's limit; the histogram's last cell), B not a
    # multiple of the workgroup size
    _run(777, 32, 20, policy=sv.ADAPT_SPEEDUP, window=16, k_min=2, k_max=32, cost=0.01, seed=3)


def test_no_lens_and_zero_depth_pass():
    _run(300, 5, 6, policy=sv.ADAPT_THRESHOLD, window=4, k_min=1, k_max=5, seed=4, lens=False)
    _run(64, 0, 3, policy=sv.ADAPT_THRESHOLD, window=4, k_min=1, k_max=5, seed=5)


def test_many_rows_grid_stride():
    # more rows than the 256 x 256 threads of the capped grid
    _run(150_000, 7, 2, policy=sv.ADAPT_SPEEDUP, window=8, k_min=1, k_max=7, cost=0.05, seed=6)


def test_empty_call_counts_itself():
    dev = torch.device("cuda:0")
    tel = sv.adapt_telemetry(dev)
    e = torch.empty(0, dtype=torch.int32, device=dev)
    sv.adapt(e, None, sv.adapt_state(0, dev), tel, K=4, k_max=4)
    torch.cuda.synchronize()
    assert sv.telemetry_counters(tel)["calls"] == 1
    assert int(tel.abs().sum()) == 1


def test_closed_loop_with_accept():
    """accept -> adapt -> next draft lengths -> accept ..., with the GPU's own
    accept outputs fed to the oracle's controller (the accept pass has its
    own parity tests)."""
    dev = torch.device("cuda:0")
    B, K, V = 64, 6, 20000
    inp = workloads.accept_inputs(B, K, V, logit_std=3.0, draft_noise=1.5, temperature=0.8, seed=21,
                                  bf16=True)
    z, q, x = inp.logits.to(dev), torch.from_numpy(inp.draft_probs).to(dev), \
        torch.from_numpy(inp.draft_tokens).to(dev)
    ws = sv.accept_workspace(B, K, V, dev)
    st_g, tel_g = sv.adapt_state(B, dev), sv.adapt_telemetry(dev)
    st_o, tel_o = C.new_state(B), C.new_telemetry()
    lens = torch.full((B,), K, dtype=torch.int32, device=dev)
    for r in range(12):
        print(f"[spec_adapt] closed loop round {r}", flush=True)
        res = sv.accept(z, q, x, lens, temperature=inp.temperature, seed=inp.seed, offset=r,
                        workspace=ws)
        nxt = sv.adapt(res.accepted, lens, st_g, tel_g, K=K, k_min=1, k_max=K, window=4,
                       policy=sv.ADAPT_SPEEDUP, draft_cost=0.05)
        torch.cuda.synchronize()
        nxt_o, st_o, tel_o = C.adapt(res.accepted.cpu().numpy(), lens.cpu().numpy(), K, st_o, tel_o,
                                     k_min=1, k_max=K, window=4, policy=C.POLICY_SPEEDUP,
                                     draft_cost=0.05)
        assert np.array_equal(nxt.cpu().numpy(), nxt_o)
        assert np.array_equal(st_g.cpu().numpy(), st_o)
        assert np.array_equal(tel_g.cpu().numpy().astype(np.uint64), tel_o)
        lens = nxt.clone()
    cnt = sv.telemetry_counters(tel_g)
    assert cnt["rows"] == 12 * B and cnt["calls"] == 12
    assert cnt["hist"].sum() == cnt["rows"]
