"""spec_accept_noalloc (the entry point that allocates nothing: its
workspace is a static device array) against spec_accept with a caller's
workspace, through the C ABI, on two calls in a row, the second smaller.
The two share their kernels, so the outputs must agree bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import speculative_decoding_verification_accept_amd as sv
from speculative_decoding_verification_accept_amd import workloads

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module")
def noalloc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # the C ABI directly: the binding only declares the argument types
    return sv.load_library().spec_accept_noalloc


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _call_noalloc(fn, z, q, x, L, T, seed, offset):
    B, K1, V = z.shape
    K = K1 - 1
    dev = z.device
    out = [torch.full((B, K1), -7, dtype=torch.int32, device=dev),
           torch.full((B,), -7, dtype=torch.int32, device=dev),
           torch.full((B, K), -7.0, dtype=torch.float32, device=dev),
           torch.full((B,), -7, dtype=torch.int32, device=dev)]
    dt = sv.SPEC_BF16 if z.dtype == torch.bfloat16 else sv.SPEC_F32
    rc = fn(_p(z), dt, _p(q), _p(x), _p(L), B, K, V, 0, float(T), seed, offset,
            _p(out[0]), _p(out[1]), _p(out[2]), _p(out[3]),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == sv.SPEC_OK, rc
    return [o.cpu().numpy() for o in out]


def _case(B, K, V, bf16, T, seed):
    inp = workloads.accept_inputs(B, K, V, logit_std=3.0, draft_noise=1.0, temperature=T,
                                  seed=seed, bf16=bf16, ragged=True, greedy=T == 0.0)
    z = inp.logits.cuda()
    q = None if inp.draft_probs is None else torch.from_numpy(inp.draft_probs).cuda()
    x = torch.from_numpy(inp.draft_tokens).cuda()
    L = torch.from_numpy(inp.draft_lens).cuda()
    return z, q, x, L, T, inp.seed


def test_noalloc_matches_spec_accept(noalloc):
    # first call: the fused step's shape (fp32 logits, V = 151936); second, smaller
    for i, (B, K, V, bf16, T) in enumerate([(32, 5, 151936, False, 0.6), (8, 3, 32000, True, 0.8),
                                            (6, 4, 5000, False, 0.0)]):
        print(f"[spec_accept_noalloc] call {i}: B={B} K={K} V={V} bf16={bf16} T={T}", flush=True)
        z, q, x, L, T, seed = _case(B, K, V, bf16, T, seed=50 + i)
        got = _call_noalloc(noalloc, z, q, x, L, T, seed, 11)
        ref = sv.accept(z, q, x, L, temperature=T, seed=seed, offset=11)
        torch.cuda.synchronize()
        for g, r in zip(got, (ref.tokens, ref.accepted, ref.p_draft, ref.status)):
            assert np.array_equal(g, r.cpu().numpy())
        assert np.all(got[1] >= 0)


def test_noalloc_rejects_oversize(noalloc):
    # a call whose workspace would exceed the static array is refused before
    # any launch: B = 2048 rows of V = 151936 (fp32) need ~160 MiB
    dev = torch.device("cuda:0")
    z = torch.zeros(1, dtype=torch.float32, device=dev)
    rc = noalloc(_p(z), sv.SPEC_F32, _p(z), _p(z), None, 2048, 5, 151936, 0, 0.5, 1, 0,
                 _p(z), _p(z), None, None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == sv.SPEC_ERR_WORKSPACE
