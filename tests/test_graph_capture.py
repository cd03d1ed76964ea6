"""The verify step's entry points inside a captured HIP graph: they allocate
nothing, launch only kernels (no memset or copy nodes), and leave their
workspaces in the state the next call expects, so a captured step replays.
Each graph is replayed several times with eager work of the same kind in
between, and every replay is compared with the eager result bit for bit.
"""
import pytest
import torch

import speculative_decoding_verification_accept_amd as sv
from speculative_decoding_verification_accept_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sv.load_library()


def _replays(capture, eager, outs, n=3):
    """Capture `capture` in a graph, then replay it n times, each after an
    eager run of `eager` (which rewrites the same outputs) and a
    synchronisation; every replay must reproduce the first eager result."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        capture()  # warm-up outside the graph, on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture()
    for k in range(n):
        eager()
        torch.cuda.synchronize()
        for o in outs:
            o.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"replay {k} differs from the eager result"


def test_verify_step_in_a_graph():
    # the step's lm-head product (a round of 192 x 512 tiles, the remaining
    # columns split along K, and the reduction of their partials) and the
    # accept pass over its logits
    dev = torch.device("cuda:0")
    B, K, V, H = 32, 5, workloads.LMHEAD_N, workloads.HIDDEN
    M = B * (K + 1)
    X, W = workloads.linear_inputs(M, H, V, seed=3, device=dev)
    logits = torch.empty(M, V, dtype=torch.float32, device=dev)
    n = sv.linear_workspace_bytes(M, V, H)
    ws_lin = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    sv.verify_linear(X, W, out=logits, workspace=ws_lin)
    z3 = logits.view(B, K + 1, V)
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    q, x, L = workloads.draft_side_device(z3, K, 1.0, 0.6, g, ragged=True)
    ws_acc = sv.accept_workspace(B, K, V, dev)
    out = sv.AcceptResult(torch.empty(B, K + 1, dtype=torch.int32, device=dev),
                          torch.empty(B, dtype=torch.int32, device=dev),
                          torch.empty(B, K, dtype=torch.float32, device=dev),
                          torch.empty(B, dtype=torch.int32, device=dev))

    def step():
        sv.verify_linear(X, W, out=logits, workspace=ws_lin)
        sv.accept(z3, q, x, L, temperature=0.6, seed=5, offset=9, workspace=ws_acc, out=out)

    _replays(step, step, [logits, out.tokens, out.accepted, out.p_draft, out.status])


@pytest.mark.parametrize("M", [8, 32])
def test_small_m_linear_in_a_graph(M):
    # the 32-row tile split in two along K, and the reduction of its partials
    dev = torch.device("cuda:0")
    H, N = workloads.HIDDEN, workloads.FFN_N
    X, W = workloads.linear_inputs(M, H, N, seed=40 + M, device=dev)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    n = sv.linear_workspace_bytes(M, N, H)
    assert n > 0  # the split-K plan needs fp32 partials
    ws = torch.empty(n, dtype=torch.uint8, device=dev)

    def run():
        sv.verify_linear(X, W, out=Y, workspace=ws)

    _replays(run, run, [Y])


def test_packed_lmhead_in_a_graph():
    # the packed-weight lm-head product the step times: two rounds of tiles,
    # the remaining tiles split along K, and the reduction of their partials
    dev = torch.device("cuda:0")
    M, H, V = 192, workloads.HIDDEN, workloads.LMHEAD_N
    X, W = workloads.linear_inputs(M, H, V, seed=45, device=dev)
    Wp = sv.pack_weight(W)
    Y = torch.empty(M, V, dtype=torch.float32, device=dev)
    n = sv.linear_packed_workspace_bytes(M, V, H)
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device=dev)

    def run():
        sv.verify_linear_packed(X, Wp, V, out=Y, workspace=ws)

    _replays(run, run, [Y])


def test_sampled_accept_in_a_graph():
    dev = torch.device("cuda:0")
    z, d, x, L = workloads.sampled_accept_device(7, dev, B=16, K=5, V=32768)
    B, K1, V = z.shape
    ws = sv.accept_sampled_workspace(B, K1 - 1, V, dev)
    out = sv.AcceptResult(torch.empty(B, K1, dtype=torch.int32, device=dev),
                          torch.empty(B, dtype=torch.int32, device=dev),
                          torch.empty(B, K1 - 1, dtype=torch.float32, device=dev),
                          torch.empty(B, dtype=torch.int32, device=dev))

    def call():
        sv.accept_sampled(z, d, x, L, temperature=0.8, top_p=0.95, min_p=0.05, seed=3, offset=1,
                          workspace=ws, out=out)

    _replays(call, call, list(out))


def test_verify_attention_in_a_graph():
    # a cache long enough to be split across workgroups: the split partials
    # and the combine launch are in the graph too
    dev = torch.device("cuda:0")
    B, K, H, Hkv, S = 2, 3, 8, 2, 6000
    ctx = [5900, 3000]
    q, kc, vc, ct, ln = workloads.attention_inputs(B, K, H, Hkv, ctx, S, seed=2, device=dev,
                                                   draft_lens=[3, 2])
    ws = torch.empty(max(sv.attention_workspace_bytes(B, K, H, Hkv, S), 1), dtype=torch.uint8, device=dev)
    out = torch.empty(B, K + 1, H, 128, dtype=torch.bfloat16, device=dev)

    def call():
        sv.verify_attention(q, kc, vc, ct, ln, out=out, workspace=ws)

    _replays(call, call, [out])
