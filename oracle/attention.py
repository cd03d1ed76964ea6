"""Oracle of verify attention: the K+1 query positions of each sequence in a
verify pass attend, causally, to the sequence's KV cache.

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; the library's
product path never does.  It shares no code with the HIP implementation.
fp64 throughout (bf16 inputs widen exactly); a library matmul serves as the
dot products.

Sources (cited by page title and section):
  [P1] "Speculative decoding and early exit: accelerated autoregressive
       decoding" (reactapp.top), section "Attention structure during
       decoding": every decode step's queries read the whole, growing key /
       value memory of the sequence (one head: Q [8, 1, 128] against K and V
       [8, 2048, 128]); section "Speculative decoding: draft first, then
       verify": one target pass processes the K+1 positions.
  [P2] "Decode is memory-bound: ~59 tok/s ceiling on an RTX 4090, and how
       speculative decoding beats it" (trefon.com), section on the ceiling:
       at long context the KV cache is read in full on every pass, on top of
       the weights.
  [P3] agentnet.co.il item, section "GEMM-M grows, a small batch suffices":
       verifying D drafts multiplies the rows the target processes by 1+D.

Readings taken where the pages are silent:
  * Scaled dot-product attention: softmax(scale * q.k) over the allowed keys,
    then the weighted sum of the values; scale is an argument (1/sqrt(d) by
    convention).
  * Query i of sequence b (i = 0 .. L_b: the token that ended the previous
    pass, then the L_b drafts) sits at position ctx_b + i, and its key and
    value are already in the cache there.  It attends to positions
    0 .. ctx_b + i (causal within the verified block).  Rows i > L_b are
    not computed; their output is zero.
  * Grouped heads: query head h reads KV head h // (H / Hkv); H = Hkv is
    plain multi-head attention as on the page.
"""
from __future__ import annotations

import numpy as np


def verify_attention(q, k_cache, v_cache, ctx_lens, draft_lens, scale: float) -> np.ndarray:
    """q [B, K+1, H, d]; k_cache, v_cache [B, Hkv, S, d]; ctx_lens [B];
    draft_lens [B] or None (every L_b = K).  Returns out [B, K+1, H, d]
    (fp64)."""
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    B, K1, H, d = q.shape
    Hkv = kc.shape[1]
    G = H // Hkv
    out = np.zeros((B, K1, H, d))
    for b in range(B):
        L = K1 - 1 if draft_lens is None else int(draft_lens[b])
        for i in range(L + 1):
            T = int(ctx_lens[b]) + i + 1           # keys 0 .. ctx_b + i
            for h in range(H):
                g = h // G
                s = scale * (kc[b, g, :T] @ q[b, i, h])
                w = np.exp(s - s.max())
                out[b, i, h] = (w @ vc[b, g, :T]) / w.sum()
    return out


def verify_attention_row(q, k_cache, v_cache, ctx_len: int, b: int, i: int, h: int,
                         scale: float) -> np.ndarray:
    """One output row (b, i, h), the same definition, for sampled checks at
    sizes where the whole oracle would take too long."""
    H = q.shape[2]
    G = H // k_cache.shape[1]
    g = h // G
    T = int(ctx_len) + i + 1
    qv = np.asarray(q[b, i, h], dtype=np.float64)
    kk = np.asarray(k_cache[b, g, :T], dtype=np.float64)
    vv = np.asarray(v_cache[b, g, :T], dtype=np.float64)
    s = scale * (kk @ qv)
    w = np.exp(s - s.max())
    return (w @ vv) / w.sum()


def kv_bytes(ctx_lens, draft_lens, K: int, Hkv: int, d: int, elem: int = 2) -> int:
    """Bytes of keys and values a verify pass must read: every cached and
    new position of every sequence, once per KV head."""
    tot = 0
    for b, c in enumerate(ctx_lens):
        L = K if draft_lens is None else int(draft_lens[b])
        tot += (int(c) + L + 1) * Hkv * d * elem * 2
    return tot
