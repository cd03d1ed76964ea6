"""CPU oracle for the speculative-decoding verification step.

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the library's
product path never does.  It shares no code with the HIP implementation.

* :func:`spec_accept` wraps ``spec_oracle.c`` (plain fp64 C, sequential loops,
  optional OpenMP over independent rows).
* :func:`verify_linear` is the fp64 reference of the verify linear layer
  Y = X W: a textbook BLAS matmul of the exactly widened bf16 operands
  [page "New technical post reveals how speculative decoding accelerates LLM
  inference" (agentnet.co.il), section "GEMM-M grows, a small batch suffices":
  every linear layer of the target sees B(1+D) rows instead of B].
* :func:`expected_tokens_per_pass` is the closed form of the expected tokens
  per verify pass [page "Decode is memory-bound ..." (trefon.com), section
  "Speculative decoding"], used by the oracle's own pins.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_oracle.c")
_LIB = os.path.join(_HERE, "libspec_oracle.so")

ROW_NONFINITE = 1
ROW_BAD_TOKEN = 2
ROW_BAD_LEN = 4
ROW_ZERO_Q = 8
ROW_RESID_ZERO = 16

NEAR_WINDOW = 1e-6

_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
             "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    lib.oracle_philox4x32_10.argtypes = [P, P, P]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_uniforms.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32,
                                    ctypes.c_uint32, P]
    lib.oracle_uniforms.restype = None
    lib.oracle_softmax.argtypes = [P, ctypes.c_int64, ctypes.c_double, P]
    lib.oracle_softmax.restype = None
    lib.oracle_set_mutation.argtypes = [ctypes.c_int]
    lib.oracle_set_mutation.restype = None
    lib.oracle_spec_accept.argtypes = [
        P, P, P, P,
        ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_double, ctypes.c_uint64, ctypes.c_uint64,
        P, P, P, P, P, P, P, ctypes.c_int]
    lib.oracle_spec_accept.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def philox4x32_10(counter, key) -> np.ndarray:
    """One Philox4x32-10 block (Salmon et al., SC'11) as 4 uint32 words."""
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    assert c.shape == (4,) and k.shape == (2,)
    out = np.zeros(4, dtype=np.uint32)
    _load().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniforms(seed: int, offset: int, row: int, pos: int) -> tuple[float, float]:
    """(u_acc, u_smp) of one (row, position): 24-bit uniforms of words 0, 1."""
    out = np.zeros(2, dtype=np.float64)
    _load().oracle_uniforms(seed, offset, row, pos, _ptr(out))
    return float(out[0]), float(out[1])


def softmax(z, temperature: float) -> np.ndarray:
    """fp64 softmax(z / T) of one position (z given as fp32 values)."""
    z = np.ascontiguousarray(z, dtype=np.float32)
    p = np.zeros(z.shape[0], dtype=np.float64)
    _load().oracle_softmax(_ptr(z), z.shape[0], float(np.float32(temperature)), _ptr(p))
    return p


def set_mutation(m: int) -> None:
    """Plant a known mistake in the oracle (0 = none); for pin tests only."""
    _load().oracle_set_mutation(int(m))


def spec_accept(logits, draft_probs, draft_tokens, draft_lens, temperature: float,
                seed: int, offset: int, row_base: int = 0, nthreads: int = 1) -> dict:
    """Batched accept/reject in fp64.

    logits       [B, K+1, V] float32 values (bf16 inputs widened exactly)
    draft_probs  [B, K, V] float32, or None when temperature == 0
    draft_tokens [B, K] int32
    draft_lens   [B] int32 or None (all K)
    temperature  the same fp32 value the GPU receives (it is rounded to fp32
                 here and widened to fp64)
    Returns a dict of numpy arrays: tokens [B, K+1] (-1 padded), accepted [B]
    (-1 for an invalid row), p_draft [B, K] (-1 where not computed), status
    [B], near_acc [B] (first near-threshold acceptance position or -1),
    near_smp [B] (1 if the categorical draw was near its threshold),
    resid_mass [B] (S_r at a rejection, else -1).
    """
    z = np.ascontiguousarray(logits, dtype=np.float32)
    assert z.ndim == 3
    B, K1, V = z.shape
    K = K1 - 1
    q = None if draft_probs is None else np.ascontiguousarray(draft_probs, dtype=np.float32)
    if q is not None:
        assert q.shape == (B, K, V), (q.shape, (B, K, V))
    x = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, K)
    L = None if draft_lens is None else np.ascontiguousarray(draft_lens, dtype=np.int32).reshape(B)
    T = float(np.float32(temperature))
    out = dict(
        tokens=np.zeros((B, K + 1), np.int32), accepted=np.zeros(B, np.int32),
        p_draft=np.zeros((B, K), np.float64), status=np.zeros(B, np.int32),
        near_acc=np.zeros(B, np.int32), near_smp=np.zeros(B, np.int32),
        resid_mass=np.zeros(B, np.float64))
    rc = _load().oracle_spec_accept(
        _ptr(z), _ptr(q), _ptr(x), _ptr(L), B, K, V, row_base, T,
        seed & (2**64 - 1), offset & (2**64 - 1),
        _ptr(out["tokens"]), _ptr(out["accepted"]), _ptr(out["p_draft"]),
        _ptr(out["status"]), _ptr(out["near_acc"]), _ptr(out["near_smp"]),
        _ptr(out["resid_mass"]), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_spec_accept rejected its arguments (rc={rc})")
    return out


def verify_linear(X, W) -> np.ndarray:
    """fp64 reference of Y = X W (X [M, K], W [K, N] given as exact fp32
    widenings of the bf16 operands)."""
    return np.asarray(X, dtype=np.float64) @ np.asarray(W, dtype=np.float64)


def verify_linear_entries(X, W, rows, cols) -> np.ndarray:
    """fp64 reference of selected entries Y[rows[i], cols[i]] only."""
    X = np.asarray(X)
    W = np.asarray(W)
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    return np.einsum("ik,ki->i", X[rows].astype(np.float64), W[:, cols].astype(np.float64))


def expected_tokens_per_pass(alpha, k):
    """Closed form of the expected tokens per verify pass when each of k
    drafts is accepted independently with probability alpha:
    (1 - alpha^(k+1)) / (1 - alpha), and k + 1 when alpha == 1."""
    alpha = np.asarray(alpha, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = (1.0 - alpha ** (k + 1)) / (1.0 - alpha)
    return np.where(alpha == 1.0, k + 1.0, e)


def expected_tokens_positional(alphas) -> float:
    """Expected emitted tokens when position i is accepted with probability
    alphas[i] (independently, stopping at the first rejection): the sum over
    j = 0..L of the product of alphas[:j].  Reduces to the closed form above
    when every alpha is equal."""
    total, prod = 0.0, 1.0
    for a in list(alphas) + [None]:
        total += prod
        if a is None:
            break
        prod *= a
    return total
