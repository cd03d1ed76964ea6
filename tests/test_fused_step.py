"""The fused verify step at its full size, end to end on the GPU, against the
oracle: the verify linear layer on the lm-head (hidden [192, 4096] bf16 x
W [4096, 151936] bf16 -> fp32 logits, with W as stored and with W packed in
the MFMA operand order, the form the benchmark times), then spec_accept on
those logits (B = 32, K = 5, T = 0.6).

Definition: page "Speculative decoding and early exit: accelerated
autoregressive decoding" (reactapp.top), section "Speculative decoding:
draft first, then verify", listing speculative_decode: the verify pass's own
target logits go straight into the accept/reject block.  Page "New technical
post reveals how speculative decoding accelerates LLM inference without
hurting accuracy" (agentnet.co.il), section "GEMM-M grows, a small batch
suffices": the verify pass is a linear layer over B(1+D) rows.

Checks:
  * every one of the 29.2 M logits against the fp64 oracle product
    (1e-2 of max(|y|, rms), relative Frobenius < 5e-3);
  * spec_accept's decisions and tokens against the oracle run on the SAME
    GPU logits: exact, except rows whose oracle draw lies within 1e-6 of its
    threshold (counted); p_i(x_i) within 1e-5 relative;
  * for information only: how often the oracle's decisions on its own fp64
    logits (rounded to fp32, as a product stored in fp32 is) differ from
    those on the GPU logits.  Different logits legitimately move draws that
    sit near a threshold, so this rate is reported, not bounded.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verification_accept_amd as sv
from speculative_decoding_verification_accept_amd import workloads
from accept_compare import compare, gpu_to_numpy
from linear_check import check_full, reference_sliced

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)
B, K, T = 32, 5, 0.6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()
    oracle.set_mutation(0)
    sv.load_library()


def _step_inputs(seed, draft_seed, ragged=False):
    dev = torch.device("cuda:0")
    V, H = workloads.LMHEAD_N, workloads.HIDDEN
    M = B * (K + 1)
    hidden, W = workloads.linear_inputs(M, H, V, seed=seed, device=dev)
    logits = torch.empty(M, V, dtype=torch.float32, device=dev)
    ws_n = sv.linear_workspace_bytes(M, V, H)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(draft_seed)
    return hidden, W, logits, ws, g


@pytest.mark.parametrize("ragged,packed", [(False, False), (True, False), (False, True)])
def test_fused_step_against_oracle(ragged, packed):
    print(f"[fused step] lm-head GEMM + spec_accept B={B} K={K} V={workloads.LMHEAD_N} T={T} "
          f"ragged={ragged} packed={packed}", flush=True)
    hidden, W, logits, ws_lin, g = _step_inputs(5, 2005 + ragged)
    if packed:
        # the benchmark's form: W stored once in the MFMA operand order
        sv.verify_linear_packed(hidden, sv.pack_weight(W), W.shape[1], out=logits)
    else:
        sv.verify_linear(hidden, W, out=logits, workspace=ws_lin)
    z3 = logits.view(B, K + 1, -1)
    q, x, L = workloads.draft_side_device(z3, K, 1.0, T, g, ragged=ragged)
    ws_acc = sv.accept_workspace(B, K, z3.shape[2], z3.device)
    res = sv.accept(z3, q, x, L, temperature=T, seed=0x5EED, offset=7, workspace=ws_acc)
    torch.cuda.synchronize()
    got = gpu_to_numpy(res)

    # the product, every element
    ref = reference_sliced(hidden, W)
    print("logits:", check_full(logits, ref, "lm-head logits"))

    # the accept pass on the GPU's own logits
    zh = z3.cpu().numpy()
    qh, xh, Lh = q.cpu().numpy(), x.cpu().numpy(), L.cpu().numpy()
    o = oracle.spec_accept(zh, qh, xh, Lh, T, 0x5EED, 7, nthreads=NTHREADS)
    st = compare(got, o, K, max_excluded_frac=0.1, label="fused step")
    print("accept on the GPU logits:", st)
    assert np.all(got["accepted"] >= 0) and np.all((got["status"] & ~sv.ROW_RESID_ZERO) == 0)
    if ragged:
        assert not np.array_equal(Lh, np.full(B, K))

    # for information: the oracle's decisions on its own logits
    zo = ref.astype(np.float32).reshape(B, K + 1, -1)
    o2 = oracle.spec_accept(zo, qh, xh, Lh, T, 0x5EED, 7, nthreads=NTHREADS)
    differ = ~(np.all(o2["tokens"] == o["tokens"], axis=1) & (o2["accepted"] == o["accepted"]))
    print(f"informational: decisions on oracle-computed logits differ from those on the GPU "
          f"logits in {int(differ.sum())} of {B} rows "
          f"(max |logit difference| {float(np.max(np.abs(zo - zh))):.3g})")


def test_fused_step_many_offsets_sampled_rows():
    # the same GPU logits through 40 further Philox offsets: more decisions
    # and draws per launch configuration, each checked against the oracle
    hidden, W, logits, ws_lin, g = _step_inputs(6, 3006)
    sv.verify_linear(hidden, W, out=logits, workspace=ws_lin)
    z3 = logits.view(B, K + 1, -1)
    q, x, L = workloads.draft_side_device(z3, K, 1.0, T, g)
    ws_acc = sv.accept_workspace(B, K, z3.shape[2], z3.device)
    outs = []
    for off in range(40):
        outs.append(gpu_to_numpy(sv.accept(z3, q, x, L, temperature=T, seed=99, offset=off,
                                           workspace=ws_acc)))
    torch.cuda.synchronize()
    zh, qh, xh, Lh = z3.cpu().numpy(), q.cpu().numpy(), x.cpu().numpy(), L.cpu().numpy()
    exact = excluded = 0
    rejects = 0
    for off, got in enumerate(outs):
        o = oracle.spec_accept(zh, qh, xh, Lh, T, 99, off, nthreads=NTHREADS)
        st = compare(got, o, K, max_excluded_frac=0.1, label=f"offset {off}")
        exact += st["exact"]
        excluded += st["excluded"]
        rejects += int(np.sum(o["accepted"] < Lh))
    print(f"40 offsets x {B} rows: {exact} exact, {excluded} excluded near a threshold, "
          f"{rejects} rejections")
    assert excluded <= 0.01 * 40 * B + 2
    assert 0 < rejects < 40 * B
