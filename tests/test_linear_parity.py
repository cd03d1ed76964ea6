"""spec_verify_linear on the GPU against the fp64 oracle (numpy matmul of
the exactly widened bf16 operands).

Tolerance: per element |y - y_ref| <= 1e-2 * max(|y_ref|, rms(Y_ref)); the
relative Frobenius error is also bounded.  A pure per-element relative test
is meaningless where y_ref ~ 0, since fp32 accumulation over K = 4096 terms
leaves an absolute error of order 1e-7 * sqrt(K) * |x||w|.
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verification_accept_amd as sv
from speculative_decoding_verification_accept_amd import workloads
from linear_check import check_full, reference_sliced

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sv.load_library()


def _check(Y, ref, label):
    Y = np.asarray(Y, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.abs(Y - ref)
    lim = TOL * np.maximum(np.abs(ref), rms)
    worst = np.argmax(err / lim)
    assert np.all(err <= lim), (label, float(err.flat[worst]), float(ref.flat[worst]), rms)
    fro = np.linalg.norm(Y - ref) / max(np.linalg.norm(ref), 1e-300)
    assert fro < 5e-3, (label, fro)
    return fro


@pytest.mark.parametrize("M,N,K", [
    (1, 128, 32), (5, 136, 40), (16, 256, 64), (17, 264, 200), (33, 1024, 256),
    (64, 384, 512), (65, 520, 1000), (130, 1032, 96), (300, 256, 520), (257, 8, 8),
    # several m-tiles through the tile remap: a grid of fewer tiles than
    # XCDs (without and with split-K), and a ragged 15-tile grid, on the
    # 128 x 128, 256 x 128 and 256 x 256 tiles
    (200, 136, 128), (300, 264, 512), (600, 392, 256), (520, 1160, 320),
    # past 512 rows with K a multiple of 32 but not of 64: the 256 x 128 tile
    (600, 392, 288),
    # the 32- and 64-row tiles: a ragged last column tile, K of 3 stages
    # (unsplit), and 17 tiles split in two along K
    (1, 1032, 128), (24, 520, 192), (32, 2056, 1024), (40, 1160, 192), (64, 2056, 1024),
    # 465-512 rows: the 256 x 256 tile over two row tiles, split in two along K
    (480, 1032, 1024),
])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_small_shapes_every_element(M, N, K, out_dtype):
    print(f"[spec_verify_linear] full check M={M} N={N} K={K} {out_dtype}", flush=True)
    X, W = workloads.linear_inputs(M, K, N, seed=M * 7 + N, device="cuda")
    Y = sv.verify_linear(X, W, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = oracle.verify_linear(X.float().cpu().numpy(), W.float().cpu().numpy())
    _check(Y.float().cpu().numpy(), ref, (M, N, K))


def _full(M, N, K, out_dtype, seed):
    X, W = workloads.linear_inputs(M, K, N, seed=seed, device="cuda")
    Y = sv.verify_linear(X, W, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return check_full(Y, reference_sliced(X, W), (M, N, K, out_dtype))


@pytest.mark.parametrize("M", workloads.sweep_ms())
def test_sweep_shapes_every_element(M):
    # the sweep's launch at full size, every output against the fp64 oracle
    print(f"[spec_verify_linear] sweep M={M} N={workloads.FFN_N} K={workloads.HIDDEN}", flush=True)
    r = _full(M, workloads.FFN_N, workloads.HIDDEN, torch.bfloat16, seed=1000 + M)
    print(f"M={M} {r}")


def test_between_sweep_sizes_every_element():
    # M = 768 takes the 256 x 256 tile in one round of 168 tiles
    print(f"[spec_verify_linear] M=768 N={workloads.FFN_N} K={workloads.HIDDEN}", flush=True)
    print(_full(768, workloads.FFN_N, workloads.HIDDEN, torch.bfloat16, seed=1768))


def test_lmhead_every_element():
    # the lm-head launch of the fused step (a round of 192 x 512 tiles, then
    # the remaining columns as 192 x 256 tiles split along K and summed by
    # the reduce)
    print("[spec_verify_linear] lm-head M=192 N=151936 K=4096 fp32", flush=True)
    print(_full(192, workloads.LMHEAD_N, workloads.HIDDEN, torch.float32, seed=5))


@pytest.mark.parametrize("M,N,K,out_dtype", [
    # 192 x 512 tiles over a partial M tile, then one remaining 256-column
    # tile (8 columns of it in range) split four ways along K
    (129, 131080, 512, torch.float32),
    # a partial last 256-column tile; K of 8 stages: the remainder unsplit
    (160, 140000, 256, torch.bfloat16),
    # exactly whole rounds of 192 x 512 tiles: no remainder launch
    (192, 131072, 1024, torch.float32),
])
def test_wide_tile_plan_every_element(M, N, K, out_dtype):
    print(f"[spec_verify_linear] wide tiles M={M} N={N} K={K} {out_dtype}", flush=True)
    print(_full(M, N, K, out_dtype, seed=M + N + K))


def test_deterministic_and_m_only():
    # equal M = B(1+D) from different (B, D) is the same GEMM: results are a
    # function of the inputs only, bit for bit across calls
    X, W = workloads.linear_inputs(32, 4096, 14336, seed=3, device="cuda")
    a = sv.verify_linear(X, W, out_dtype=torch.bfloat16)
    b = sv.verify_linear(X, W, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # row m of the product depends on row m of X only
    c = sv.verify_linear(X[:8].contiguous(), W, out_dtype=torch.float32)
    d = sv.verify_linear(X, W, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.allclose(c, d[:8], rtol=0, atol=1e-3)
