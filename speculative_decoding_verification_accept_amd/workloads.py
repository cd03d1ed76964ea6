"""Seeded synthetic inputs for the verification step.

This module is shared by the tests, the benchmark and the CPU oracle's
callers.  It holds none of the verification arithmetic: it draws target
logits, synthesises what a draft model would hand to the verifier (draft
probabilities through a library softmax of noisy logits, draft tokens through
numpy's own categorical sampler, per-row draft lengths) and draws the inputs
of the verify linear layer.  The draft side is outside the verification step
[page "Speculative decoding and early exit: accelerated autoregressive
decoding" (reactapp.top), section "Speculative decoding: draft first, then
verify", listing `speculative_decode`, draft phase].

Draw order per workload (numpy PCG64, ``default_rng(seed)``): target logits,
draft-logit noise, draft lengths, draft tokens.  bf16 values are produced by
round-to-nearest-even from fp32 on the CPU.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import scipy.special
import torch


@dataclass
class AcceptInputs:
    """One batch of accept/reject inputs, host-resident.

    logits: torch CPU tensor [B, K+1, V], float32 or bfloat16
    draft_probs: float32 numpy [B, K, V] or None (greedy)
    draft_tokens: int32 numpy [B, K]
    draft_lens: int32 numpy [B]
    """
    logits: torch.Tensor
    draft_probs: np.ndarray | None
    draft_tokens: np.ndarray
    draft_lens: np.ndarray
    temperature: float
    seed: int
    offset: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.logits.shape[0]

    @property
    def K(self):
        return self.logits.shape[1] - 1

    @property
    def V(self):
        return self.logits.shape[2]

    def logits_f32(self) -> np.ndarray:
        """Exact fp32 values of the logits (bf16 widens without rounding)."""
        return self.logits.float().numpy()


def draft_probs_from_logits(draft_logits: np.ndarray, temperature: float) -> np.ndarray:
    """What a draft model hands over: softmax(draft_logits / T) as fp32,
    computed by scipy in fp64 (the draft side, not the verifier)."""
    return scipy.special.softmax(
        np.asarray(draft_logits, np.float64) / temperature, axis=-1).astype(np.float32)


def sample_draft_tokens(rng: np.random.Generator, q: np.ndarray) -> np.ndarray:
    """Draft tokens x ~ q for each leading index of q [..., V], via numpy's
    categorical sampler (the draft model's own draw)."""
    lead = q.shape[:-1]
    V = q.shape[-1]
    flat = q.reshape(-1, V)
    out = np.empty(flat.shape[0], np.int32)
    for r in range(flat.shape[0]):
        p = flat[r].astype(np.float64)
        out[r] = rng.choice(V, p=p / p.sum())
    return out.reshape(lead)


def _to_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)


def accept_inputs(B: int, K: int, V: int, *, logit_std: float, draft_noise: float,
                  temperature: float, seed: int, bf16: bool = False,
                  ragged: bool = False, greedy: bool = False,
                  philox_seed: int | None = None, offset: int = 0) -> AcceptInputs:
    """Generic recipe shared by the named workloads below.

    Target logits z ~ N(0, logit_std^2) [B, K+1, V] (fp32, or rounded to
    bf16); draft logits = z + N(0, draft_noise^2) at the K drafted positions;
    q = softmax(draft / T); draft tokens x ~ q.  ragged: L_b ~ U{1..K}.
    greedy (T = 0): draft tokens are the draft logits' argmax, q is None.
    """
    rng = np.random.default_rng(seed)
    z = rng.normal(0.0, logit_std, size=(B, K + 1, V)).astype(np.float32)
    logits = _to_bf16(z) if bf16 else torch.from_numpy(z)
    z_seen = logits.float().numpy()
    noise = rng.normal(0.0, draft_noise, size=(B, K, V)).astype(np.float32)
    draft_logits = z_seen[:, :K, :] + noise
    lens = (rng.integers(1, K + 1, size=B) if ragged else np.full(B, K)).astype(np.int32)
    if greedy:
        q = None
        tokens = np.argmax(draft_logits, axis=-1).astype(np.int32)
    else:
        q = draft_probs_from_logits(draft_logits, temperature)
        tokens = sample_draft_tokens(rng, q)
    return AcceptInputs(logits, q, tokens.reshape(B, K), lens, float(temperature),
                        seed=philox_seed if philox_seed is not None else 1000 + seed,
                        offset=offset, meta=dict(seed=seed))


def replicated_inputs(rounds: int, K: int, V: int, *, logit_std: float, draft_noise: float,
                      temperature: float, seed: int, lens: int | None = None) -> AcceptInputs:
    """Many independent rounds of one distribution: the logits and q are drawn
    once ([K+1, V] and [K, V]) and replicated over `rounds` rows; each row
    gets its own draft tokens x_i ~ q_i (and its own Philox stream through
    its row index)."""
    rng = np.random.default_rng(seed)
    z = rng.normal(0.0, logit_std, size=(K + 1, V)).astype(np.float32)
    noise = rng.normal(0.0, draft_noise, size=(K, V)).astype(np.float32)
    q1 = draft_probs_from_logits(z[:K] + noise, temperature)
    tokens = np.empty((rounds, K), np.int32)
    for i in range(K):
        p = q1[i].astype(np.float64)
        tokens[:, i] = rng.choice(V, size=rounds, p=p / p.sum())
    logits = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(z, (rounds, K + 1, V))))
    q = np.ascontiguousarray(np.broadcast_to(q1, (rounds, K, V)))
    L = np.full(rounds, K if lens is None else lens, np.int32)
    return AcceptInputs(logits, q, tokens, L, float(temperature), seed=1000 + seed,
                        meta=dict(seed=seed, z=z, q=q1))


# --- named workloads --------------------------------------------------------

def small_accept(rounds: int = 2000, seed: int = 1) -> AcceptInputs:
    """CPU-sized: B=1, K=4, V=1000, z ~ N(0, 2^2) fp32, draft noise
    N(0, 0.5^2), T=1.0; `rounds` independent rounds as rows."""
    return replicated_inputs(rounds, 4, 1000, logit_std=2.0, draft_noise=0.5,
                             temperature=1.0, seed=seed)


def tiny_vocab(rounds: int = 1_000_000, K: int = 4, seed: int = 11) -> AcceptInputs:
    """V=8 variant for the distribution-equality tests."""
    return replicated_inputs(rounds, K, 8, logit_std=2.0, draft_noise=0.5,
                             temperature=1.0, seed=seed)


def mid_accept(seed: int = 2, greedy: bool = False) -> AcceptInputs:
    """B=8, K=4, V=32000, fp32 z ~ N(0, 3^2), draft noise N(0, 1), T=0.6
    (T=0 and argmax drafts for the greedy variant)."""
    return accept_inputs(8, 4, 32000, logit_std=3.0, draft_noise=1.0,
                         temperature=0.0 if greedy else 0.6, seed=seed, greedy=greedy)


def large_accept(seed: int = 3, B: int = 64) -> AcceptInputs:
    """B=64, K=7, V=128256, bf16 z ~ N(0, 3^2), draft noise N(0, 1.5^2),
    T=0.8, ragged L_b ~ U{1..7}."""
    return accept_inputs(B, 7, 128256, logit_std=3.0, draft_noise=1.5,
                         temperature=0.8, seed=seed, bf16=True, ragged=True)


# --- verify linear layer ----------------------------------------------------

HIDDEN = 4096
FFN_N = 14336
LMHEAD_N = 151936
SWEEP_BD = [(1, 0), (1, 3), (1, 7), (8, 0), (8, 3), (8, 7),
            (32, 0), (32, 3), (32, 7), (128, 0), (128, 3), (128, 7)]


def sweep_ms():
    """M = B(1+D) for B in {1, 8, 32, 128} and D in {0, 3, 7}."""
    return sorted({b * (1 + d) for b, d in SWEEP_BD})


def linear_inputs(M: int, K: int, N: int, seed: int, device="cpu",
                  x_std: float = 1.0, w_std: float = 0.02):
    """bf16 X [M, K] ~ N(0, x_std^2) and W [K, N] ~ N(0, w_std^2), drawn with
    torch's seeded generator on `device` (fp32 normals rounded to bf16)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    X = (torch.randn(M, K, generator=g, device=device) * x_std).to(torch.bfloat16)
    W = (torch.randn(K, N, generator=g, device=device) * w_std).to(torch.bfloat16)
    return X, W


# --- device-resident synthesis for the benchmark ------------------------------

def draft_side_device(target_logits: torch.Tensor, K: int, draft_noise: float,
                      temperature: float, gen: torch.Generator, ragged: bool = False):
    """Draft side of a verify step synthesised on the GPU with torch ops: draft
    logits = target logits (first K positions) + N(0, draft_noise^2), q =
    softmax(draft / T) in fp32, x ~ q by torch.multinomial, and optional
    ragged lengths L_b ~ U{1..K}.  target_logits is [B, K+1, V]."""
    B, K1, V = target_logits.shape
    dl = target_logits[:, :K, :].float()
    dl = dl + draft_noise * torch.randn(dl.shape, generator=gen, device=dl.device)
    q = torch.softmax(dl.double() / temperature, dim=-1).float().contiguous()
    x = torch.multinomial(q.view(-1, V), 1, generator=gen).view(B, K).to(torch.int32)
    if ragged:
        L = torch.randint(1, K + 1, (B,), generator=gen, device=dl.device, dtype=torch.int32)
    else:
        L = torch.full((B,), K, dtype=torch.int32, device=dl.device)
    return q, x.contiguous(), L


def large_accept_device(seed: int, device, B: int = 64, K: int = 7, V: int = 128256):
    """Device-resident inputs with the recipe of large_accept(): bf16 target
    logits ~ N(0, 3^2), draft noise N(0, 1.5^2), T = 0.8, ragged L_b."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = (3.0 * torch.randn(B, K + 1, V, generator=g, device=device)).to(torch.bfloat16)
    q, x, L = draft_side_device(z, K, 1.5, 0.8, g, ragged=True)
    return z, q, x, L


# --- verify attention ------------------------------------------------------------
# Shapes: the pages' decode example is one head of Q [8, 1, 128] against a
# 2048-token cache, 32 heads (multi-head); the grouped variant uses 8 KV heads
# for 32 query heads, head dim 128, the attention of the model whose linear
# layer is the 4096 x 14336 sweep.
ATTN_HEAD_DIM = 128


def attention_inputs(B: int, K: int, H: int, Hkv: int, ctx_lens, S: int, seed: int, device,
                     draft_lens=None):
    """bf16 q [B, K+1, H, 128] and caches [B, Hkv, S, 128] ~ N(0, 1), drawn
    with torch's seeded generator on `device`; positions past each
    sequence's ctx_b + L_b + 1 hold the same draws (never read)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    q = torch.randn(B, K + 1, H, ATTN_HEAD_DIM, generator=g, device=device).to(torch.bfloat16)
    kc = torch.randn(B, Hkv, S, ATTN_HEAD_DIM, generator=g, device=device).to(torch.bfloat16)
    vc = torch.randn(B, Hkv, S, ATTN_HEAD_DIM, generator=g, device=device).to(torch.bfloat16)
    ctx = torch.as_tensor(np.asarray(ctx_lens, dtype=np.int32), device=device)
    lens = None if draft_lens is None else torch.as_tensor(np.asarray(draft_lens, dtype=np.int32),
                                                           device=device)
    return q, kc, vc, ctx, lens


def sampled_accept_device(seed: int, device, B: int = 64, K: int = 7, V: int = 128256,
                          noise: float = 1.5):
    """Device-resident inputs for accept/reject with the draft as logits:
    bf16 target logits ~ N(0, 3^2), bf16 draft logits = target + N(0, noise^2),
    ragged L_b ~ U{1..K}; each draft token is the draft's top logit (always
    inside the draft's filtered distribution)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = (3.0 * torch.randn(B, K + 1, V, generator=g, device=device)).to(torch.bfloat16)
    d = (z[:, :K].float() + noise * torch.randn(B, K, V, generator=g, device=device)).to(torch.bfloat16)
    x = d.float().argmax(-1).to(torch.int32)
    L = torch.randint(1, K + 1, (B,), generator=g, device=device, dtype=torch.int32)
    return z, d, x, L
