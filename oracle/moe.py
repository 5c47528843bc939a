"""The Flint-shaped MoE layer, stated plainly in float64 (oracle).

TEST INFRASTRUCTURE: see the package docstring for who may use it.

What the pages fix:
  * Layer shape -- "Day-0 Support for Flint on vLLM", section "Model
    architecture", third bullet (and the arex-research write-up, section
    "Flint 是什么", second paragraph): 256 routed experts scored with a
    sigmoid, the top 6 taken, plus one shared expert that is always on;
    hidden size 2048; a pre-norm residual stack.
  * Only the selected experts' weights are read ("Optimizations", second
    bullet): skipping an unselected expert is exact because its combine
    weight is zero, so the oracle simply loops over the selected ones.
  * Weight-only W4A16 with BF16 activations, kernels rounding where the
    reference rounds ("Model architecture", paragraph after the bullets;
    "Optimizations", fourth bullet): every BF16 rounding point below is
    explicit.

Readings where the pages are silent (each is listed in the design notes):
  * expert MLP = SwiGLU: y = W_d (SiLU(W_g z) * W_u z), SiLU(z) = z/(1+e^-z);
  * router: BF16 weights, logits accumulated without rounding, no bias, no
    scaling factor, no expert groups; top-k by descending score, ties to the
    lower expert index; combine weight = raw sigmoid score, or the score
    divided by the sum of the selected scores ("renorm");
  * shared expert weight 1, no gate; rounding points: BF16(g), BF16(u),
    BF16(SiLU(g)), BF16(SiLU(g)*u); the down projections and the weighted
    sum stay unrounded and the layer output is rounded once;
  * RMSNorm (decode step only): xn = BF16(BF16(x / sqrt(mean(x^2) + eps)) *
    gamma); residual update x <- BF16(x + out).
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional

import numpy as np

from .bf16 import round_bf16
from .formats import decode_source_matrix


# ----------------------------------------------------------------- pieces --

def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def rmsnorm(x, gamma, eps: float = 1e-6):
    """Pre-norm RMSNorm with the two BF16 rounding points; x [.., H]."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return round_bf16(round_bf16(x / np.sqrt(ms + eps)) * np.asarray(gamma, dtype=np.float64))


def topk_select(scores, k: int):
    """Indices of the k largest scores of one token, ordered by descending
    score with ties to the lower index, and the gap between the k-th and the
    (k+1)-th largest score (inf when k equals the number of experts).  A NaN
    score (from a NaN router weight) ranks below every number."""
    s = np.asarray(scores, dtype=np.float64)
    s = np.where(np.isnan(s), -np.inf, s)
    order = np.lexsort((np.arange(s.size), -s))     # primary: -s, then index
    idx = order[:k]
    gap = float(s[order[k - 1]] - s[order[k]]) if k < s.size else float("inf")
    return idx.astype(np.int64), gap


def expert_ffn(z, w_gate, w_up, w_down):
    """SwiGLU expert on one token with the BF16 rounding points.  Returns
    the unrounded down projection and the intermediates (g, u, h)."""
    z = np.asarray(z, dtype=np.float64)
    g = round_bf16(w_gate @ z)
    u = round_bf16(w_up @ z)
    a = round_bf16(silu(g))
    h = round_bf16(a * u)
    return w_down @ h, (g, u, h)


# ---------------------------------------------------------------- weights --

@dataclasses.dataclass
class ExpertSet:
    """Float64 weights of one MoE layer, decoded on demand.

    ``expert(e)`` returns (W_gate [I][H], W_up [I][H], W_down [H][I]) for a
    routed expert e, or for the shared expert when e is None (None is also
    returned for the whole triple when the layer has no shared expert)."""

    router: np.ndarray                                  # [E][H] float64 (BF16 values)
    n_experts: int
    _loader: Callable[[Optional[int]], Optional[tuple]]
    _cache: dict = dataclasses.field(default_factory=dict)

    def expert(self, e: Optional[int]):
        key = -1 if e is None else int(e)
        if key not in self._cache:
            self._cache[key] = self._loader(e)
        return self._cache[key]


def nvfp4_expert_set(router, gate, up, down, gscale, sh_gate=None, sh_up=None, sh_down=None,
                     sh_gscale=None, layout: str = "interleaved") -> ExpertSet:
    """ExpertSet over source NVFP4 super-blocks (numpy uint8):
    gate/up [E][I][H/64][36], down [E][H][I/64][36], gscale [E][3]
    (gate, up, down FP32 scales per expert); the shared expert's arrays
    have a leading dimension of 1."""
    gscale = np.asarray(gscale, dtype=np.float64)

    def load(e):
        if e is None:
            if sh_gate is None:
                return None
            s = np.asarray(sh_gscale, dtype=np.float64).reshape(3)
            return (decode_source_matrix(sh_gate[0], layout, s[0]),
                    decode_source_matrix(sh_up[0], layout, s[1]),
                    decode_source_matrix(sh_down[0], layout, s[2]))
        return (decode_source_matrix(gate[e], layout, gscale[e, 0]),
                decode_source_matrix(up[e], layout, gscale[e, 1]),
                decode_source_matrix(down[e], layout, gscale[e, 2]))

    router = np.asarray(router, dtype=np.float64)
    return ExpertSet(router=router, n_experts=router.shape[0], _loader=load)


# ------------------------------------------------------------------ layer --

@dataclasses.dataclass
class Routing:
    logits: np.ndarray      # [B][E]
    scores: np.ndarray      # [B][E] sigmoid
    idx: np.ndarray         # [B][K] int64
    weight: np.ndarray      # [B][K] combine weights
    gap: np.ndarray         # [B] k-th minus (k+1)-th score


def route(xn, router, top_k: int, renorm: bool, forced_idx=None) -> Routing:
    """Router GEMV, sigmoid and top-k for a batch of tokens xn [B][H]."""
    xn = np.atleast_2d(np.asarray(xn, dtype=np.float64))
    logits = xn @ np.asarray(router, dtype=np.float64).T
    scores = sigmoid(logits)
    B = xn.shape[0]
    idx = np.zeros((B, top_k), dtype=np.int64)
    w = np.zeros((B, top_k))
    gap = np.zeros(B)
    for t in range(B):
        sel, gap[t] = topk_select(scores[t], top_k)
        if forced_idx is not None:
            sel = np.asarray(forced_idx[t], dtype=np.int64)
        idx[t] = sel
        s_sel = scores[t, sel]
        w[t] = s_sel / s_sel.sum() if renorm else s_sel
    return Routing(logits, scores, idx, w, gap)


def moe_layer(xn, experts: ExpertSet, top_k: int, renorm: bool, forced_idx=None):
    """The MoE layer on BF16 inputs xn [B][H]: per token,
    out = BF16( sum_k w_k * E_{idx_k}(xn) + E_shared(xn) ).
    Returns (out [B][H] float64 holding BF16 values, Routing)."""
    xn = np.atleast_2d(np.asarray(xn, dtype=np.float64))
    r = route(xn, experts.router, top_k, renorm, forced_idx)
    out = np.zeros_like(xn)
    shared = experts.expert(None)
    for t in range(xn.shape[0]):
        acc = np.zeros(xn.shape[1])
        for k in range(top_k):
            y, _ = expert_ffn(xn[t], *experts.expert(int(r.idx[t, k])))
            acc = acc + r.weight[t, k] * y
        if shared is not None:
            y, _ = expert_ffn(xn[t], *shared)
            acc = acc + y
        out[t] = round_bf16(acc)
    return out, r


def moe_sublayer(x, gamma, experts: ExpertSet, top_k: int, renorm: bool, eps: float = 1e-6,
                 forced_idx=None):
    """Pre-norm residual MoE sublayer: x <- BF16(x + MoE(RMSNorm(x)))."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    out, r = moe_layer(rmsnorm(x, gamma, eps), experts, top_k, renorm, forced_idx)
    return round_bf16(x + out), r


def dense_mlp(xn, w_gate, w_up, w_down):
    """Dense SwiGLU MLP (one expert, weight 1) with the output rounded."""
    xn = np.atleast_2d(np.asarray(xn, dtype=np.float64))
    return np.stack([round_bf16(expert_ffn(z, w_gate, w_up, w_down)[0]) for z in xn])


def dense_sublayer(x, gamma, w_gate, w_up, w_down, eps: float = 1e-6):
    """Pre-norm residual dense sublayer: x <- BF16(x + MLP(RMSNorm(x)))."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return round_bf16(x + dense_mlp(rmsnorm(x, gamma, eps), w_gate, w_up, w_down))


def prefill(x, experts: ExpertSet, top_k: int, renorm: bool, tokens=None):
    """Prefill is the decode layer applied to every token independently
    (the permutation by expert, grouped GEMM and un-permutation reach the
    same per-token result).  ``tokens`` restricts the work to a sample."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    sel = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    return moe_layer(x[sel], experts, top_k, renorm)


def expert_histogram(idx, n_experts: int):
    """Number of (token, slot) pairs routed to each expert."""
    return np.bincount(np.asarray(idx).reshape(-1), minlength=n_experts)
