"""Per-head Q/K RMSNorm, rotary position embedding and the KV-cache write of
one attention layer's projected heads (oracle).

TEST INFRASTRUCTURE: see the package docstring for who may use it.

What the pages fix:
  * "Day-0 Support for Flint on vLLM", section "Model architecture", the
    attention bullets: grouped-query attention with 32 query heads and 4 KV
    heads of dimension 128, and a per-head RMSNorm of Q and K; 35 layers
    attend to a sliding window with RoPE, the other 14 to the full context
    with no positional encoding;
  * the same section, paragraph after the bullets: the KV cache is BF16;
  * section "Optimizations", first bullet: the Q/K norm, RoPE and the
    KV-cache write are one step (one kernel instead of three).

Readings where the pages are silent (each is listed in the design notes):
  * the per-head norm has the library's RMSNorm rounding points,
    BF16(BF16(x / sqrt(mean(x^2) + eps)) * gamma), over one head's values,
    with one gamma per role (q, k) shared by all heads of that role;
  * the norm comes first, then RoPE (the order the pages list them in);
  * RoPE rotates the pairs (x_i, x_{i+d/2}), i < d/2 ("rotate half"), by the
    angle of the caller's cos/sin table row at the token's position: each
    output is the exact rotation of the BF16 normalised inputs, rounded to
    BF16 once;
  * the fused projection row is [q heads | k heads | v heads]; V goes to the
    cache unchanged, K after its norm and RoPE; cache layout
    [slot][kv head][d]; a negative slot writes nothing (a padding token).
"""
from __future__ import annotations

import numpy as np

from .bf16 import round_bf16
from .moe import rmsnorm


def head_rmsnorm(x, gamma, eps: float = 1e-6):
    """RMSNorm of each head (last axis = one head's d values) with the two
    BF16 rounding points."""
    return rmsnorm(x, gamma, eps)


def rope_rotate_half(x, cos, sin):
    """Rotary embedding of heads x [.., d] by the angles whose cosines and
    sines are cos, sin [.., d/2] (broadcast over the heads): pair i is
    (x_i, x_{i+d/2}) and becomes (x_i c_i - x_{i+d/2} s_i, x_{i+d/2} c_i +
    x_i s_i).  Unrounded float64."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def qk_norm_rope_kv(qkv, n_q: int, n_kv: int, d: int, positions, slots, gamma_q, gamma_k, cos_sin,
                    k_cache, v_cache, eps: float = 1e-6, rope: bool = True):
    """The fused step for T tokens.

    qkv       [T][(n_q + 2 n_kv) d] projected heads (BF16 values)
    positions [T] row of cos_sin per token (used when rope)
    slots     [T] KV-cache row per token; negative: not written
    cos_sin   [P][d] table rows: cos of the d/2 angles, then their sines
    k_cache, v_cache [S][n_kv][d], updated in place

    Returns q [T][n_q][d] (BF16 values as float64)."""
    qkv = np.asarray(qkv, dtype=np.float64)
    T = qkv.shape[0]
    q = qkv[:, : n_q * d].reshape(T, n_q, d)
    k = qkv[:, n_q * d: (n_q + n_kv) * d].reshape(T, n_kv, d)
    v = qkv[:, (n_q + n_kv) * d:].reshape(T, n_kv, d)
    qn = head_rmsnorm(q, gamma_q, eps)
    kn = head_rmsnorm(k, gamma_k, eps)
    if rope:
        cs = np.asarray(cos_sin, dtype=np.float64)[np.asarray(positions)]      # [T][d]
        c = cs[:, None, : d // 2]
        s = cs[:, None, d // 2:]
        qn = round_bf16(rope_rotate_half(qn, c, s))
        kn = round_bf16(rope_rotate_half(kn, c, s))
    for t in range(T):
        if slots[t] >= 0:
            k_cache[slots[t]] = kn[t]
            v_cache[slots[t]] = v[t]
    return qn
