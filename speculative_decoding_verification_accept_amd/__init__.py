"""MI355X-native speculative-decoding verification step.

Thin Python binding over ``libspecverify.so`` (C ABI in include/spec_verify.h).
It only marshals arguments: tensors must already live on the GPU, every step
of the computation runs in the library's HIP kernels, and there is no CPU
fallback -- if the library is missing, calls raise.

* :func:`accept` -- batched accept/reject pass (``spec_accept``)
* :func:`verify_linear` -- verify linear layer Y = X W (``spec_verify_linear``)
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple

import torch

from . import _build

SPEC_F32 = 0
SPEC_BF16 = 1
SPEC_OK = 0
SPEC_ERR_INVALID_ARG = -1
SPEC_ERR_WORKSPACE = -2
SPEC_ERR_HIP = -3
ROW_NONFINITE = 1
ROW_BAD_TOKEN = 2
ROW_BAD_LEN = 4
ROW_ZERO_Q = 8
ROW_RESID_ZERO = 16
ROW_STALLED = 32
MAX_DRAFT = 255

# (name, restype, argtypes) for every entry point declared in the header
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
ABI = [
    ("spec_accept_workspace_bytes", ctypes.c_size_t, [_I64, ctypes.c_int, _I64]),
    ("spec_accept", ctypes.c_int,
     [_P, ctypes.c_int, _P, _P, _P, _I64, ctypes.c_int, _I64, _I64, ctypes.c_float, _U64, _U64,
      _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    ("spec_verify_linear_workspace_bytes", ctypes.c_size_t, [_I64, _I64, _I64]),
    ("spec_verify_linear", ctypes.c_int,
     [_P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]),
    ("spec_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("spec_abi_version", ctypes.c_int, []),
]

_lib = None


class SpecError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {status_string(code)} ({code})")
        self.code = code


def library_path() -> str:
    return _build.LIB_PATH


def load_library():
    """Load libspecverify.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    for name, res, args in ABI:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load_library().spec_status_string(int(code)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_dev(name, t, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def accept_workspace_bytes(B: int, K: int, V: int) -> int:
    return int(load_library().spec_accept_workspace_bytes(B, K, V))


def accept_workspace(B: int, K: int, V: int, device) -> torch.Tensor:
    """A zero-filled workspace for spec_accept (the library keeps it zeroed
    from call to call; reuse it for calls of the same or smaller size)."""
    return torch.zeros(max(accept_workspace_bytes(B, K, V), 1), dtype=torch.uint8, device=device)


def linear_workspace_bytes(M: int, N: int, Kd: int) -> int:
    return int(load_library().spec_verify_linear_workspace_bytes(M, N, Kd))


class AcceptResult(NamedTuple):
    tokens: torch.Tensor     # [B, K+1] int32, -1 padded
    accepted: torch.Tensor   # [B] int32 (a_b; -1 for an invalid row)
    p_draft: torch.Tensor    # [B, K] float32 (p_i(x_i) for i < L_b, else -1)
    status: torch.Tensor     # [B] int32 row status bits


def accept(target_logits, draft_probs, draft_tokens, draft_lens=None, *, temperature: float,
           seed: int, offset: int = 0, row_base: int = 0, workspace=None, out=None,
           stream=None) -> AcceptResult:
    """Batched accept/reject (``spec_accept``) on the current stream.

    target_logits [B, K+1, V] float32 or bfloat16; draft_probs [B, K, V]
    float32 (None iff temperature == 0); draft_tokens [B, K] int32;
    draft_lens [B] int32 or None.  Returns device tensors; they are valid
    once the stream has synchronised.
    """
    _check_dev("target_logits", target_logits, ndim=3)
    if target_logits.dtype == torch.float32:
        dt = SPEC_F32
    elif target_logits.dtype == torch.bfloat16:
        dt = SPEC_BF16
    else:
        raise TypeError("target_logits must be float32 or bfloat16")
    B, K1, V = target_logits.shape
    K = K1 - 1
    dev = target_logits.device
    if draft_probs is not None:
        _check_dev("draft_probs", draft_probs, torch.float32, 3)
        if tuple(draft_probs.shape) != (B, K, V):
            raise ValueError("draft_probs must be [B, K, V]")
    _check_dev("draft_tokens", draft_tokens, torch.int32, 2)
    if tuple(draft_tokens.shape) != (B, K):
        raise ValueError("draft_tokens must be [B, K]")
    if draft_lens is not None:
        _check_dev("draft_lens", draft_lens, torch.int32, 1)
        if draft_lens.shape[0] != B:
            raise ValueError("draft_lens must be [B]")
    lib = load_library()
    if out is None:
        out = AcceptResult(torch.empty(B, K + 1, dtype=torch.int32, device=dev),
                           torch.empty(B, dtype=torch.int32, device=dev),
                           torch.empty(B, K, dtype=torch.float32, device=dev),
                           torch.empty(B, dtype=torch.int32, device=dev))
    if workspace is None:
        workspace = accept_workspace(B, K, V, dev)
    rc = lib.spec_accept(
        _ptr(target_logits), dt, _ptr(draft_probs), _ptr(draft_tokens), _ptr(draft_lens),
        B, K, V, row_base, float(temperature), seed & (2**64 - 1), offset & (2**64 - 1),
        _ptr(out.tokens), _ptr(out.accepted), _ptr(out.p_draft), _ptr(out.status),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != SPEC_OK:
        raise SpecError("spec_accept", rc)
    return out


def verify_linear(X, W, *, out=None, out_dtype=torch.float32, workspace=None, stream=None):
    """Y = X W with bf16 operands and fp32 accumulation (``spec_verify_linear``).

    X [M, Kd] bfloat16, W [Kd, N] bfloat16 (input-major), Y [M, N] float32 or
    bfloat16.
    """
    _check_dev("X", X, torch.bfloat16, 2)
    _check_dev("W", W, torch.bfloat16, 2)
    M, Kd = X.shape
    Kd2, N = W.shape
    if Kd != Kd2:
        raise ValueError("X and W inner dimensions differ")
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=X.device)
    _check_dev("out", out, None, 2)
    if out.dtype == torch.float32:
        yd = SPEC_F32
    elif out.dtype == torch.bfloat16:
        yd = SPEC_BF16
    else:
        raise TypeError("out must be float32 or bfloat16")
    lib = load_library()
    need = lib.spec_verify_linear_workspace_bytes(M, N, Kd)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.spec_verify_linear(_ptr(X), _ptr(W), _ptr(out), yd, M, N, Kd, _ptr(workspace),
                                nbytes, _stream(stream))
    if rc != SPEC_OK:
        raise SpecError("spec_verify_linear", rc)
    return out
