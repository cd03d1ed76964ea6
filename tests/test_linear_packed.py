"""spec_pack_weight and spec_verify_linear_packed on the GPU against the fp64
oracle: the verify linear layer Y = X W with W stored in the MFMA operand
order.

Definition: page "New technical post reveals how speculative decoding
accelerates LLM inference without hurting accuracy" (agentnet.co.il),
sections "The formula behind the speedup" and "GEMM-M grows, a small batch
suffices" (a linear layer over M = B(1+D) rows).  The packed layout is this
library's own storage format: the packing is checked byte for byte against
the layout written out from its definition in numpy; the product, element
by element against the oracle (tolerance of linear_check: 1e-2 of
max(|y|, rms), relative Frobenius error below 5e-3).

The shapes reach the 64-, 128- and 192-row tiles, several row tiles, split
and unsplit plans (the split sums four columns per thread when N is a
multiple of 4, one otherwise), ragged rows and columns, and the lm-head in the launch
configuration the benchmark times (two whole rounds of tiles, the remaining
tiles split three ways along K, their reduce).
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verification_accept_amd as sv
from speculative_decoding_verification_accept_amd import workloads
from linear_check import check_full, reference_sliced

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()
    oracle.set_mutation(0)
    sv.load_library()


def _layout_reference(W: np.ndarray) -> np.ndarray:
    """The packed layout from its definition: block (s, c), record 64 h + l,
    element j = W[32 s + 8 (l // 16) + j, 32 c + 16 h + l % 16], zero past N."""
    K, N = W.shape
    C = (N + 31) // 32
    Wz = np.zeros((K, C * 32), W.dtype)
    Wz[:, :N] = W
    s, c, h, l, j = np.meshgrid(np.arange(K // 32), np.arange(C), np.arange(2), np.arange(64),
                                np.arange(8), indexing="ij")
    return Wz[32 * s + 8 * (l // 16) + j, 32 * c + 16 * h + l % 16]


@pytest.mark.parametrize("K,N", [(64, 1), (128, 70), (192, 256), (256, 1032)])
def test_pack_matches_the_layout_definition(K, N):
    print(f"[packed] pack K={K} N={N}", flush=True)
    _, W = workloads.linear_inputs(1, K, N, seed=K + N, device="cuda")
    Wp = sv.pack_weight(W)
    torch.cuda.synchronize()
    assert Wp.numel() == sv.packed_weight_bytes(K, N) == K * ((N + 31) // 32) * 64
    got = Wp.cpu().numpy().view(np.uint16).reshape(K // 32, (N + 31) // 32, 2, 64, 8)
    ref = _layout_reference(W.cpu().view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(got, ref)


SHAPES = [
    (1, 8, 64), (5, 70, 128), (17, 300, 192), (64, 520, 576), (65, 1032, 256),
    (100, 264, 640), (128, 2056, 512), (129, 1000, 64), (192, 2056, 1024), (193, 520, 128),
    (250, 777, 320), (400, 264, 512), (40, 777, 512), (3, 514, 1024), (7, 1, 64), (1000, 264, 128),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_small_shapes_every_element(M, N, K):
    print(f"[packed] M={M} N={N} K={K}", flush=True)
    X, W = workloads.linear_inputs(M, K, N, seed=M * 7 + N + K, device="cuda")
    Wp = sv.pack_weight(W)
    ref = oracle.verify_linear(X.float().cpu().numpy(), W.float().cpu().numpy())
    for dt in (torch.float32, torch.bfloat16):
        Y = sv.verify_linear_packed(X, Wp, N, out_dtype=dt)
        torch.cuda.synchronize()
        check_full(Y, ref, (M, N, K, dt))


@pytest.mark.parametrize("M", [64, 256, 512])
def test_sweep_shapes_every_element(M):
    # the verify GEMM's weight [4096, 14336] at row counts of the sweep: split
    # plans (M <= 128) and several 192-row tiles (M = 256, 512)
    K, N = workloads.HIDDEN, workloads.FFN_N
    print(f"[packed] sweep M={M} N={N} K={K}", flush=True)
    X, W = workloads.linear_inputs(M, K, N, seed=M, device="cuda")
    Y = sv.verify_linear_packed(X, sv.pack_weight(W), N, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    print(check_full(Y, reference_sliced(X, W), ("sweep", M)))


def test_lmhead_every_element():
    M, K, N = 192, workloads.HIDDEN, workloads.LMHEAD_N
    print(f"[packed] lm-head M={M} N={N} K={K}", flush=True)
    X, W = workloads.linear_inputs(M, K, N, seed=11, device="cuda")
    Wp = sv.pack_weight(W)
    Y = sv.verify_linear_packed(X, Wp, N)
    Y2 = sv.verify_linear_packed(X, Wp, N)
    Yu = sv.verify_linear(X, W)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)  # deterministic: fixed summation order
    print(check_full(Y, reference_sliced(X, W), "lm-head"))
    # the stored-layout product sums in another order; they agree to fp32 rounding
    d = (Y - Yu).abs().max().item()
    print(f"max |packed - unpacked| = {d:.3g}")
    assert d < 1e-3 * Yu.abs().max().item()


def test_workspace_and_empty():
    M, K, N = 64, 576, 520
    X, W = workloads.linear_inputs(M, K, N, seed=3, device="cuda")
    Wp = sv.pack_weight(W)
    lib = sv.load_library()
    need = lib.spec_verify_linear_packed_workspace_bytes(M, N, K)
    assert need > 0  # 3 tiles: split along K
    Y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    rc = lib.spec_verify_linear_packed(X.data_ptr(), Wp.data_ptr(), Y.data_ptr(), sv.SPEC_F32, M, N, K,
                                       None, 0, None)
    assert rc == sv.SPEC_ERR_WORKSPACE
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    rc = lib.spec_verify_linear_packed(X.data_ptr(), Wp.data_ptr(), Y.data_ptr(), sv.SPEC_F32, M, N, K,
                                       small.data_ptr(), small.numel(), None)
    assert rc == sv.SPEC_ERR_WORKSPACE
    out = sv.verify_linear_packed(X[:0], Wp, N)
    assert out.shape == (0, N)
