"""Per-head Q/K RMSNorm, rotary position embedding and the KV-cache write of
one attention layer's projected heads, and decode attention with learned
sinks over a sliding window or the full context (oracle).

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

Decode attention.  The pages fix: "Model architecture", first two bullets
(35 layers see a 513-token window, the current token and the 512 before it;
14 layers see the whole context; GQA 32/4, head dimension 128; learned
attention sinks) and "Optimizations", fifth bullet (a decode attention
kernel with sinks and sliding windows).  Readings:
  * query head h reads KV head h // (n_q / n_kv) (consecutive query heads
    share a KV head);
  * score = scale * (q . k); a sink is one learned logit per query head that
    joins the softmax's normaliser and carries no value:
        out = sum_p exp(s_p) v_p / (sum_p exp(s_p) + exp(sink));
  * a sequence of context length L (its newest token included) attends to
    positions max(0, L - W) .. L - 1 for a window W, or 0 .. L - 1 when W is
    0 (the full-context layers); position p lives in cache row
    base + (p mod C), for the sequence's first row ``base`` and C rows per
    sequence (C >= the attended span; a ring buffer when C is the window).
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


def attended_positions(length: int, window: int):
    """Positions a decode token at context length ``length`` attends to."""
    lo = max(0, length - window) if window > 0 else 0
    return np.arange(lo, length)


def decode_attention(q, k_cache, v_cache, seq_base, seq_len, ring: int, window: int, sinks, scale: float,
                     with_abs: bool = False):
    """One decode token per sequence.

    q        [B][n_q][d] queries (after norm and RoPE)
    k_cache, v_cache [S][n_kv][d]
    seq_base [B] first cache row of each sequence; seq_len [B] its length
    ring     cache rows per sequence; window 0 for the whole context
    sinks    [n_q] one logit per query head

    Returns out [B][n_q][d] (float64, unrounded); with ``with_abs`` also the
    same mixture taken of |v| (sum_p w_p |v_p|, w the softmax weights), the
    scale of the rounding error of any mixture of the values."""
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    B, n_q, d = q.shape
    n_kv = kc.shape[1]
    group = n_q // n_kv
    out = np.zeros((B, n_q, d))
    mix_abs = np.zeros((B, n_q, d))
    for b in range(B):
        pos = attended_positions(int(seq_len[b]), window)
        rows = int(seq_base[b]) + pos % ring
        for h in range(n_q):
            g = h // group
            k = kc[rows, g]                           # [n][d]
            v = vc[rows, g]
            s = scale * (k @ q[b, h])                 # [n]
            m = max(np.max(s), float(sinks[h]))
            e = np.exp(s - m)
            z = np.sum(e) + np.exp(float(sinks[h]) - m)
            w = e / z
            out[b, h] = w @ v
            mix_abs[b, h] = w @ np.abs(v)
    return (out, mix_abs) if with_abs else out
