"""MI355X-native speculative-decoding verification step.

Thin Python binding over ``libspecverify.so`` (C ABI in include/spec_verify.h).
It only marshals arguments: tensors must already live on the GPU, every step
of the computation runs in the library's HIP kernels, and there is no CPU
fallback -- if the library is missing, calls raise.

* :func:`accept` -- batched accept/reject pass (``spec_accept``)
* :func:`accept_sampled` -- the same with the draft as logits and the
  sampler's top-p / min-p filters (``spec_accept_sampled``)
* :func:`verify_linear` -- verify linear layer Y = X W (``spec_verify_linear``)
* :func:`verify_attention` -- the verify pass's attention, K+1 causal queries
  per sequence against its KV cache (``spec_verify_attention``)
* :func:`adapt` -- acceptance telemetry and next draft depth (``spec_adapt``)
* :func:`plan_depth` -- draft depth per batch size from a measured verify-cost
  curve (``spec_plan_depth``, a host function)
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple

import numpy as np
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
ADAPT_MAX_K = 32
ADAPT_STATE_BYTES = 64
ADAPT_TELEMETRY_WORDS = 1200
ADAPT_THRESHOLD = 0
ADAPT_SPEEDUP = 1

# (name, restype, argtypes) for every entry point declared in the header
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
ABI = [
    ("spec_accept_workspace_bytes", ctypes.c_size_t, [_I64, ctypes.c_int, _I64]),
    ("spec_accept", ctypes.c_int,
     [_P, ctypes.c_int, _P, _P, _P, _I64, ctypes.c_int, _I64, _I64, ctypes.c_float, _U64, _U64,
      _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    ("spec_accept_noalloc", ctypes.c_int,
     [_P, ctypes.c_int, _P, _P, _P, _I64, ctypes.c_int, _I64, _I64, ctypes.c_float, _U64, _U64,
      _P, _P, _P, _P, _P]),
    ("spec_accept_sampled_workspace_bytes", ctypes.c_size_t, [_I64, ctypes.c_int, _I64]),
    ("spec_accept_sampled", ctypes.c_int,
     [_P, _P, ctypes.c_int, _P, _P, _I64, ctypes.c_int, _I64, _I64, ctypes.c_float,
      ctypes.c_float, ctypes.c_float, ctypes.c_float, _U64, _U64, _P, _P, _P, _P, _P,
      ctypes.c_size_t, _P]),
    ("spec_verify_linear_workspace_bytes", ctypes.c_size_t, [_I64, _I64, _I64]),
    ("spec_verify_linear", ctypes.c_int,
     [_P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]),
    ("spec_packed_weight_bytes", ctypes.c_size_t, [_I64, _I64]),
    ("spec_pack_weight", ctypes.c_int, [_P, _P, _I64, _I64, _P]),
    ("spec_verify_linear_packed_workspace_bytes", ctypes.c_size_t, [_I64, _I64, _I64]),
    ("spec_verify_linear_packed", ctypes.c_int,
     [_P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]),
    ("spec_verify_attention_workspace_bytes", ctypes.c_size_t,
     [_I64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _I64]),
    ("spec_verify_attention", ctypes.c_int,
     [_P, _P, _P, _P, _P, _I64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _I64, ctypes.c_int,
      ctypes.c_float, _P, ctypes.c_int, _P, _P, ctypes.c_size_t, _P]),
    ("spec_adapt_state_bytes", ctypes.c_size_t, [_I64]),
    ("spec_adapt_telemetry_bytes", ctypes.c_size_t, []),
    ("spec_adapt", ctypes.c_int,
     [_P, _P, _I64, ctypes.c_int, _P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
      ctypes.c_int, ctypes.c_double, ctypes.c_double, _P]),
    ("spec_plan_depth", ctypes.c_int,
     [_P, _P, ctypes.c_int, _P, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double,
      _P, _P, _P, _P]),
    ("spec_debug_set_wait_bound", ctypes.c_int, [ctypes.c_int]),
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


def set_wait_bound(polls: int) -> None:
    """Polls of a row's decision before a spec_accept workgroup gives up
    (``spec_debug_set_wait_bound``; 0 restores the default).  For tests of
    the give-up path."""
    rc = load_library().spec_debug_set_wait_bound(int(polls))
    if rc != SPEC_OK:
        raise SpecError("spec_debug_set_wait_bound", rc)


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


def accept_sampled_workspace(B: int, K: int, V: int, device) -> torch.Tensor:
    """A zero-filled workspace for spec_accept_sampled (kept zeroed by the
    library from call to call)."""
    n = int(load_library().spec_accept_sampled_workspace_bytes(B, K, V))
    return torch.zeros(max(n, 1), dtype=torch.uint8, device=device)


def accept_sampled(target_logits, draft_logits, draft_tokens, draft_lens=None, *,
                   temperature: float, draft_temperature=None, top_p: float = 1.0,
                   min_p: float = 0.0, seed: int, offset: int = 0, row_base: int = 0,
                   workspace=None, out=None, stream=None) -> AcceptResult:
    """Accept/reject with the draft as logits and the sampler's filters
    (``spec_accept_sampled``): p' and q' are top-p / min-p filtered tempered
    softmaxes of target_logits [B, K+1, V] and draft_logits [B, K, V] (same
    dtype, float32 or bfloat16)."""
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
    _check_dev("draft_logits", draft_logits, target_logits.dtype, 3)
    if tuple(draft_logits.shape) != (B, K, V):
        raise ValueError("draft_logits must be [B, K, V]")
    _check_dev("draft_tokens", draft_tokens, torch.int32, 2)
    if draft_lens is not None:
        _check_dev("draft_lens", draft_lens, torch.int32, 1)
    if draft_temperature is None:
        draft_temperature = temperature
    if out is None:
        out = AcceptResult(torch.empty(B, K + 1, dtype=torch.int32, device=dev),
                           torch.empty(B, dtype=torch.int32, device=dev),
                           torch.empty(B, K, dtype=torch.float32, device=dev),
                           torch.empty(B, dtype=torch.int32, device=dev))
    if workspace is None:
        workspace = accept_sampled_workspace(B, K, V, dev)
    rc = load_library().spec_accept_sampled(
        _ptr(target_logits), _ptr(draft_logits), dt, _ptr(draft_tokens), _ptr(draft_lens), B, K,
        V, row_base, float(temperature), float(draft_temperature), float(top_p), float(min_p),
        seed & (2**64 - 1), offset & (2**64 - 1), _ptr(out.tokens), _ptr(out.accepted),
        _ptr(out.p_draft), _ptr(out.status), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != SPEC_OK:
        raise SpecError("spec_accept_sampled", rc)
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


def linear_packed_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(load_library().spec_verify_linear_packed_workspace_bytes(M, N, K))


def packed_weight_bytes(K: int, N: int) -> int:
    """Bytes of W [K, N] in the packed layout (``spec_packed_weight_bytes``;
    0 for an unsupported shape)."""
    return int(load_library().spec_packed_weight_bytes(K, N))


def pack_weight(W, *, out=None, stream=None):
    """W [K, N] bfloat16 (input-major) rewritten into the MFMA operand order
    (``spec_pack_weight``); returns a uint8 tensor of packed_weight_bytes(K, N)."""
    _check_dev("W", W, torch.bfloat16, 2)
    K, N = W.shape
    nbytes = packed_weight_bytes(K, N)
    if nbytes == 0:
        raise ValueError(f"unsupported shape for the packed layout: K={K}, N={N} "
                         "(K must be a positive multiple of 64)")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    _check_dev("out", out)
    if out.numel() * out.element_size() < nbytes:
        raise ValueError("out is smaller than the packed weight")
    rc = load_library().spec_pack_weight(_ptr(W), _ptr(out), K, N, _stream(stream))
    if rc != SPEC_OK:
        raise SpecError("spec_pack_weight", rc)
    return out


def verify_linear_packed(X, Wp, N: int, *, out=None, out_dtype=torch.float32, workspace=None,
                         stream=None):
    """Y = X W with W packed by pack_weight (``spec_verify_linear_packed``).

    X [M, K] bfloat16, Wp the packed W [K, N], Y [M, N] float32 or bfloat16.
    """
    _check_dev("X", X, torch.bfloat16, 2)
    _check_dev("Wp", Wp)
    M, K = X.shape
    nbytes = packed_weight_bytes(K, N)
    if nbytes == 0 or Wp.numel() * Wp.element_size() < nbytes:
        raise ValueError("Wp does not hold a packed weight of this K and N")
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
    need = lib.spec_verify_linear_packed_workspace_bytes(M, N, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.spec_verify_linear_packed(_ptr(X), _ptr(Wp), _ptr(out), yd, M, N, K, _ptr(workspace),
                                       wsb, _stream(stream))
    if rc != SPEC_OK:
        raise SpecError("spec_verify_linear_packed", rc)
    return out


# --- verify attention ---------------------------------------------------------

ATTN_HEAD_DIM = 128
ATTN_MAX_ROWS = 32


def attention_workspace_bytes(B: int, K: int, H: int, Hkv: int, S: int) -> int:
    return int(load_library().spec_verify_attention_workspace_bytes(B, K, H, Hkv, S))


def verify_attention(q, k_cache, v_cache, ctx_lens, draft_lens=None, *, scale=None, out=None,
                     out_dtype=torch.float32, status=None, workspace=None, stream=None):
    """Attention of a verify pass (``spec_verify_attention``).

    q [B, K+1, H, 128] bf16; k_cache, v_cache [B, Hkv, S, 128] bf16;
    ctx_lens [B] int32 (cached tokens before the pass); draft_lens [B] int32
    or None.  Query i of sequence b attends to cache positions 0 .. ctx_b + i.
    Returns out [B, K+1, H, 128] (rows past L_b are zero).
    """
    _check_dev("q", q, torch.bfloat16, 4)
    _check_dev("k_cache", k_cache, torch.bfloat16, 4)
    _check_dev("v_cache", v_cache, torch.bfloat16, 4)
    B, K1, H, d = q.shape
    _, Hkv, S, d2 = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[0] != B or d2 != d:
        raise ValueError("k_cache and v_cache must be [B, Hkv, S, head_dim]")
    _check_dev("ctx_lens", ctx_lens, torch.int32, 1)
    if draft_lens is not None:
        _check_dev("draft_lens", draft_lens, torch.int32, 1)
    if out is None:
        out = torch.empty(B, K1, H, d, dtype=out_dtype, device=q.device)
    _check_dev("out", out, None, 4)
    if out.dtype == torch.float32:
        od = SPEC_F32
    elif out.dtype == torch.bfloat16:
        od = SPEC_BF16
    else:
        raise TypeError("out must be float32 or bfloat16")
    if status is not None:
        _check_dev("status", status, torch.int32, 1)
    if scale is None:
        scale = float(d) ** -0.5
    lib = load_library()
    need = lib.spec_verify_attention_workspace_bytes(B, K1 - 1, H, Hkv, S)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.spec_verify_attention(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_lens), _ptr(draft_lens), B, K1 - 1, H,
        Hkv, S, d, float(scale), _ptr(out), od, _ptr(status), _ptr(workspace), nbytes,
        _stream(stream))
    if rc != SPEC_OK:
        raise SpecError("spec_verify_attention", rc)
    return out


# --- controller ---------------------------------------------------------------

# telemetry word offsets (the layout spec_adapt documents)
TEL_ROWS, TEL_INVALID, TEL_DRAFTED, TEL_TESTED, TEL_ACCEPTED, TEL_EMITTED, TEL_CALLS = range(7)
TEL_TESTED_AT = 8
TEL_ACCEPTED_AT = TEL_TESTED_AT + ADAPT_MAX_K
TEL_DEPTH_HIST = TEL_ACCEPTED_AT + ADAPT_MAX_K
TEL_HIST = TEL_DEPTH_HIST + ADAPT_MAX_K + 1


def adapt_state(B: int, device) -> torch.Tensor:
    """Zeroed per-row controller records ([B, 64] bytes): no history yet."""
    return torch.zeros(B, ADAPT_STATE_BYTES, dtype=torch.uint8, device=device)


def adapt_telemetry(device) -> torch.Tensor:
    """A zeroed telemetry block (int64 view of the uint64 counters)."""
    return torch.zeros(ADAPT_TELEMETRY_WORDS, dtype=torch.int64, device=device)


def adapt(accepted, draft_lens, state, telemetry, *, K: int, k_min: int = 1, k_max: int,
          window: int = 8, policy: int = ADAPT_THRESHOLD, accept_floor: float = 0.35,
          draft_cost: float = 0.0, out=None, stream=None) -> torch.Tensor:
    """Acceptance telemetry and the next draft length per row (``spec_adapt``).

    accepted [B] int32 (``accept(...).accepted``); draft_lens [B] int32 or
    None (every row verified K drafts); state [B, 64] uint8 and telemetry
    [1200] int64 are updated in place.  Returns next_lens [B] int32.
    """
    _check_dev("accepted", accepted, torch.int32, 1)
    B = accepted.shape[0]
    if draft_lens is not None:
        _check_dev("draft_lens", draft_lens, torch.int32, 1)
        if draft_lens.shape[0] != B:
            raise ValueError("draft_lens must be [B]")
    _check_dev("state", state, torch.uint8, 2)
    if tuple(state.shape) != (B, ADAPT_STATE_BYTES):
        raise ValueError("state must be [B, 64] uint8")
    _check_dev("telemetry", telemetry, torch.int64, 1)
    if telemetry.shape[0] != ADAPT_TELEMETRY_WORDS:
        raise ValueError("telemetry must hold 1200 words")
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=accepted.device)
    _check_dev("out", out, torch.int32, 1)
    rc = load_library().spec_adapt(
        _ptr(accepted), _ptr(draft_lens), B, K, _ptr(state), _ptr(telemetry), _ptr(out),
        k_min, k_max, window, policy, float(accept_floor), float(draft_cost), _stream(stream))
    if rc != SPEC_OK:
        raise SpecError("spec_adapt", rc)
    return out


def telemetry_counters(telemetry) -> dict:
    """The telemetry block's counters by name (host copy; no arithmetic)."""
    t = telemetry.detach().cpu().numpy().astype(np.uint64)
    k = ADAPT_MAX_K
    return {
        "rows": int(t[TEL_ROWS]), "invalid_rows": int(t[TEL_INVALID]),
        "drafted": int(t[TEL_DRAFTED]), "tested": int(t[TEL_TESTED]),
        "accepted": int(t[TEL_ACCEPTED]), "emitted": int(t[TEL_EMITTED]),
        "calls": int(t[TEL_CALLS]),
        "tested_at": t[TEL_TESTED_AT:TEL_TESTED_AT + k].astype(np.int64),
        "accepted_at": t[TEL_ACCEPTED_AT:TEL_ACCEPTED_AT + k].astype(np.int64),
        "depth_hist": t[TEL_DEPTH_HIST:TEL_DEPTH_HIST + k + 1].astype(np.int64),
        "hist": t[TEL_HIST:TEL_HIST + (k + 1) ** 2].astype(np.int64).reshape(k + 1, k + 1),
    }


class DepthPlan(NamedTuple):
    best_depth: np.ndarray     # [nB] int32
    speedup: np.ndarray        # [nB, d_max+1]
    tokens_per_s: np.ndarray   # [nB, d_max+1] (whole batch)
    pareto: np.ndarray         # [nB, d_max+1] bool


def plan_depth(m_pts, t_us, batches, *, d_max: int, alpha: float, draft_cost: float = 0.0) -> DepthPlan:
    """Draft depth per batch size from a measured verify-cost curve
    (``spec_plan_depth``, host code): m_pts rows (ascending) with their pass
    times t_us in microseconds."""
    m = np.ascontiguousarray(m_pts, dtype=np.int64)
    t = np.ascontiguousarray(t_us, dtype=np.float64)
    b = np.ascontiguousarray(batches, dtype=np.int64)
    if m.shape != t.shape or m.ndim != 1:
        raise ValueError("m_pts and t_us must be 1-D of equal length")
    nb, nd = b.shape[0], d_max + 1
    best = np.zeros(nb, np.int32)
    sp = np.zeros((nb, nd))
    rate = np.zeros((nb, nd))
    par = np.zeros((nb, nd), np.uint8)
    c = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    rc = load_library().spec_plan_depth(c(m), c(t), m.shape[0], c(b), nb, d_max, float(alpha),
                                        float(draft_cost), c(best), c(sp), c(rate), c(par))
    if rc != SPEC_OK:
        raise SpecError("spec_plan_depth", rc)
    return DepthPlan(best, sp, rate, par.astype(bool))
