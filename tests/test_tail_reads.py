"""Reads past the end of an operand: every kernel must stay inside its
operands, or read zeros where it steps past them.

Each operand is a view into a larger allocation whose tail, right after the
operand, is filled with NaN.  That memory is mapped, so a kernel that read
past an operand would not fault here, but a value it took from the tail
would turn its outputs into NaN.  The GEMM shapes reach every tile plan
(the strip kernel, the 32-, 64-, 128-, 256- and 256x256-row tiles) with
ragged rows and columns, and put the last k-stage of the register-staged
tile past K (K not a multiple of its 64-deep stage); the other shapes put
the last round of the sampler-filter row reader past the row (V not a
multiple of a round), on the last row of the logits.
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verification_accept_amd as sv
from oracle import sampled as S
from speculative_decoding_verification_accept_amd import workloads
from linear_check import check_full

pytestmark = pytest.mark.gpu

TAIL = 1 << 20  # elements of NaN after each operand


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()
    oracle.set_mutation(0)
    sv.load_library()


def _nan_tailed(t: torch.Tensor) -> torch.Tensor:
    """A copy of t at the start of an allocation whose remaining TAIL
    elements are NaN (the view is contiguous and 256-byte aligned)."""
    buf = torch.full((t.numel() + TAIL,), float("nan"), dtype=t.dtype, device=t.device)
    v = buf[: t.numel()].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("M,N,K", [(65, 520, 1000), (300, 256, 520), (257, 8, 8), (40, 1032, 200),
                                   (130, 264, 96), (8, 1032, 1024), (24, 520, 200), (48, 1160, 576),
                                   (100, 1032, 576), (300, 1032, 512), (480, 520, 512)])
def test_gemm_operands_nan_tailed(M, N, K):
    print(f"[tail reads] spec_verify_linear M={M} N={N} K={K}", flush=True)
    X, W = workloads.linear_inputs(M, K, N, seed=M + N + K, device="cuda")
    Xt, Wt = _nan_tailed(X), _nan_tailed(W)
    for dt in (torch.float32, torch.bfloat16):
        Y = sv.verify_linear(Xt, Wt, out_dtype=dt)
        torch.cuda.synchronize()
        assert torch.isfinite(Y).all(), (M, N, K, dt)
        ref = oracle.verify_linear(X.float().cpu().numpy(), W.float().cpu().numpy())
        check_full(Y, ref, (M, N, K, dt))


@pytest.mark.parametrize("M,N,K", [(5, 70, 128), (65, 1032, 576), (130, 300, 64), (200, 520, 512)])
def test_packed_gemm_operands_nan_tailed(M, N, K):
    print(f"[tail reads] spec_verify_linear_packed M={M} N={N} K={K}", flush=True)
    X, W = workloads.linear_inputs(M, K, N, seed=M + N + K, device="cuda")
    Wp = sv.pack_weight(W)
    Wpt = torch.full((Wp.numel() + 2 * TAIL,), 0xFF, dtype=torch.uint8, device="cuda")  # bf16 NaN
    Wpt = Wpt[: Wp.numel()]
    Wpt.copy_(Wp)
    Xt = _nan_tailed(X)
    for dt in (torch.float32, torch.bfloat16):
        Y = sv.verify_linear_packed(Xt, Wpt, N, out_dtype=dt)
        torch.cuda.synchronize()
        assert torch.isfinite(Y).all(), (M, N, K, dt)
        ref = oracle.verify_linear(X.float().cpu().numpy(), W.float().cpu().numpy())
        check_full(Y, ref, (M, N, K, dt))


@pytest.mark.parametrize("V,bf16", [(20000, True), (12291, False), (8200, True), (40000, False)])
@pytest.mark.parametrize("top_p,min_p", [(0.95, 0.05), (0.9, 0.0), (1.0, 0.05)])
def test_sampled_rows_nan_tailed(V, bf16, top_p, min_p):
    print(f"[tail reads] spec_accept_sampled V={V} bf16={bf16} top_p={top_p} min_p={min_p}", flush=True)
    B, K, T = 3, 2, 0.8
    rng = np.random.default_rng(V)
    z = rng.normal(0, 2.0, (B, K + 1, V)).astype(np.float32)
    d = (z[:, :K] + rng.normal(0, 0.5, (B, K, V))).astype(np.float32)
    dt = torch.bfloat16 if bf16 else torch.float32
    zt = torch.from_numpy(z).to(dt).cuda()
    dtt = torch.from_numpy(d).to(dt).cuda()
    zh, dh = zt.float().cpu().numpy(), dtt.float().cpu().numpy()
    x = np.zeros((B, K), np.int32)
    for b in range(B):
        for i in range(K):
            q = S.filtered(dh[b, i], T, float(np.float32(top_p)), float(np.float32(min_p)))[0]
            x[b, i] = rng.choice(V, p=q / q.sum())
    L = np.full(B, K, np.int32)
    res = sv.accept_sampled(_nan_tailed(zt), _nan_tailed(dtt), torch.from_numpy(x).cuda(),
                            torch.from_numpy(L).cuda(), temperature=T, top_p=top_p, min_p=min_p,
                            seed=4, offset=1)
    torch.cuda.synchronize()
    st = res.status.cpu().numpy()
    assert not np.any(st & (S.ROW_NONFINITE | S.ROW_ZERO_Q)), st
    o = S.spec_accept_sampled(zh, dh, x, L, T, T, top_p, min_p, 4, 1)
    ok = ~o["near"]
    assert np.array_equal(res.accepted.cpu().numpy()[ok], o["accepted"][ok])
    assert np.array_equal(res.tokens.cpu().numpy()[ok], o["tokens"][ok])


@pytest.mark.parametrize("V,bf16", [(20000, True), (12291, False)])
def test_accept_rows_nan_tailed(V, bf16):
    print(f"[tail reads] spec_accept V={V} bf16={bf16}", flush=True)
    inp = workloads.accept_inputs(4, 3, V, logit_std=3.0, draft_noise=1.0, temperature=0.7,
                                  seed=V, bf16=bf16, ragged=True)
    z = _nan_tailed(inp.logits.cuda())
    q = _nan_tailed(torch.from_numpy(inp.draft_probs).cuda())
    res = sv.accept(z, q, torch.from_numpy(inp.draft_tokens).cuda(),
                    torch.from_numpy(inp.draft_lens).cuda(), temperature=0.7, seed=inp.seed,
                    offset=0)
    torch.cuda.synchronize()
    o = oracle.spec_accept(inp.logits_f32(), inp.draft_probs, inp.draft_tokens, inp.draft_lens,
                           0.7, inp.seed, 0)
    assert not np.any(res.status.cpu().numpy() & 1)
    near = (o["near_acc"] >= 0) | (o["near_smp"] > 0)
    same = (res.accepted.cpu().numpy() == o["accepted"]) & np.all(
        res.tokens.cpu().numpy() == o["tokens"], axis=1)
    assert np.all(same | near)
