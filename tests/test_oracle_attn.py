"""Pins of the attention-side oracle (oracle/attn.py): per-head Q/K RMSNorm,
rotate-half RoPE and the KV-cache write, against a hand-derived example,
closed forms and properties of rotations that any correct implementation
satisfies ("Day-0 Support for Flint on vLLM", "Model architecture" and
"Optimizations")."""
import os

import numpy as np

from oracle import attn
from oracle.bf16 import round_bf16


def _golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "qk_norm_rope_small.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    vec = lambda s: np.array([float.fromhex(v) if "x" in v else float(v) for v in s.split(",")])
    return rows, vec


def test_golden_small_heads():
    rows, vec = _golden()
    assert len(rows) == 2
    d = 4
    table = np.array([[0.0, 1.0, 1.0, 0.0], [float.fromhex("0x1.333334p-1"), 1.0, float.fromhex("0x1.99999ap-1"), 0.0]])
    qkv = np.stack([np.concatenate([vec(r[3]), vec(r[4]), vec(r[5])]) for r in rows])
    pos = [int(r[1]) for r in rows]
    slots = [int(r[2]) for r in rows]
    kc = np.full((4, 1, d), 7.0)
    vc = np.full((4, 1, d), 7.0)
    q = attn.qk_norm_rope_kv(qkv, 1, 1, d, pos, slots, np.ones(d), np.array([1.0, 1.0, 2.0, 1.0]), table, kc, vc)
    for t, r in enumerate(rows):
        np.testing.assert_array_equal(q[t, 0], vec(r[6]))
        if slots[t] >= 0:
            np.testing.assert_array_equal(kc[slots[t], 0], vec(r[7]))
            np.testing.assert_array_equal(vc[slots[t], 0], vec(r[8]))
    untouched = [s for s in range(4) if s not in slots]
    assert np.all(kc[untouched] == 7.0) and np.all(vc[untouched] == 7.0)


def test_angle_zero_is_the_norm_alone():
    """cos 1, sin 0: RoPE is the identity, so the result is the head norm
    (and the no-RoPE variant gives the same)."""
    rng = np.random.default_rng(1)
    d, n_q, n_kv, T = 128, 4, 2, 3
    qkv = round_bf16(rng.standard_normal((T, (n_q + 2 * n_kv) * d)))
    gq = round_bf16(1 + 0.1 * rng.standard_normal(d))
    gk = round_bf16(1 + 0.1 * rng.standard_normal(d))
    table = np.concatenate([np.ones((1, d // 2)), np.zeros((1, d // 2))], axis=1)
    kc = np.zeros((T, n_kv, d))
    vc = np.zeros((T, n_kv, d))
    q = attn.qk_norm_rope_kv(qkv, n_q, n_kv, d, [0] * T, list(range(T)), gq, gk, table, kc, vc)
    want_q = attn.head_rmsnorm(qkv[:, : n_q * d].reshape(T, n_q, d), gq)
    np.testing.assert_array_equal(q, want_q)
    np.testing.assert_array_equal(kc, attn.head_rmsnorm(qkv[:, n_q * d: (n_q + n_kv) * d].reshape(T, n_kv, d), gk))
    np.testing.assert_array_equal(vc, qkv[:, (n_q + n_kv) * d:].reshape(T, n_kv, d))
    kc2 = np.zeros_like(kc)
    vc2 = np.zeros_like(vc)
    q2 = attn.qk_norm_rope_kv(qkv, n_q, n_kv, d, [5] * T, list(range(T)), gq, gk, None, kc2, vc2, rope=False)
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(kc2, kc)


def _angles(n_pos, d, base=10000.0):
    # a textbook frequency ladder, written out here for the property tests
    inv = base ** (-np.arange(0, d, 2) / d)
    return np.arange(n_pos)[:, None] * inv[None, :]


def test_rotation_properties():
    """Unrounded rotate-half RoPE: pair norms are kept, a rotation by a
    then by -a is the identity, and the dot product of a rotated query and
    key depends only on their position difference."""
    rng = np.random.default_rng(2)
    d = 128
    ang = _angles(64, d)
    x = rng.standard_normal(d)
    y = attn.rope_rotate_half(x, np.cos(ang[37]), np.sin(ang[37]))
    h = d // 2
    np.testing.assert_allclose(x[:h] ** 2 + x[h:] ** 2, y[:h] ** 2 + y[h:] ** 2, rtol=1e-12, atol=1e-12)
    back = attn.rope_rotate_half(y, np.cos(-ang[37]), np.sin(-ang[37]))
    np.testing.assert_allclose(back, x, rtol=0, atol=1e-12)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    rot = lambda v, p: attn.rope_rotate_half(v, np.cos(ang[p]), np.sin(ang[p]))
    a = rot(q, 20) @ rot(k, 13)
    b = rot(q, 40) @ rot(k, 33)
    c = rot(q, 7) @ rot(k, 0)
    np.testing.assert_allclose([a, b], [c, c], rtol=1e-10)


def test_pairing_is_rotate_half():
    """Pair i is (x_i, x_{i+d/2}): a one-hot x_j moves only into x_{j+d/2}
    (j < d/2), by the rotation [[c, -s], [s, c]]."""
    d = 8
    cos = np.array([1.0, 0.0, 1.0, 1.0])
    sin = np.array([0.0, 1.0, 0.0, 0.0])
    x = np.zeros(d)
    x[1] = 1.0
    np.testing.assert_array_equal(attn.rope_rotate_half(x, cos, sin), [0, 0, 0, 0, 0, 1, 0, 0])
    x = np.zeros(d)
    x[5] = 1.0
    np.testing.assert_array_equal(attn.rope_rotate_half(x, cos, sin), [0, -1, 0, 0, 0, 0, 0, 0])


def test_head_norm_is_per_head_and_scale_free():
    """Each head is normalised on its own values: with eps = 0, scaling one
    head by a power of two leaves every head's result unchanged (x / rms is
    then exactly scale free), and heads do not mix."""
    rng = np.random.default_rng(3)
    d, n = 128, 5
    x = round_bf16(rng.standard_normal((n, d)))
    g = round_bf16(1 + 0.1 * rng.standard_normal(d))
    base = attn.head_rmsnorm(x, g, 0.0)
    x2 = x.copy()
    x2[2] *= 8.0
    np.testing.assert_array_equal(attn.head_rmsnorm(x2, g, 0.0), base)
    for i in range(n):
        np.testing.assert_array_equal(attn.head_rmsnorm(x[i:i + 1], g, 0.0)[0], base[i])


def test_fused_row_layout_q_then_k_then_v():
    """The projection row is [q heads | k heads | v heads]: constants planted
    per segment land in q, the K cache and the V cache respectively."""
    d, n_q, n_kv = 128, 3, 2
    row = np.concatenate([np.full(n_q * d, 2.0), np.full(n_kv * d, 4.0), np.full(n_kv * d, 0.5)])[None, :]
    kc = np.zeros((1, n_kv, d))
    vc = np.zeros((1, n_kv, d))
    q = attn.qk_norm_rope_kv(row, n_q, n_kv, d, [0], [0], np.ones(d), np.full(d, 2.0), None, kc, vc, rope=False)
    np.testing.assert_array_equal(q, np.ones((1, n_q, d)))              # a constant head normalises to 1
    np.testing.assert_array_equal(kc, np.full((1, n_kv, d), 2.0))     # then times gamma_k
    np.testing.assert_array_equal(vc, np.full((1, n_kv, d), 0.5))


# ---------------------------------------------------------------- decode attention

def _attn_golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "decode_attention_small.txt")
    cases, cur = [], None
    for ln in open(path):
        ln = ln.strip()
        if not ln or ln.startswith("#"):
            continue
        key, *vals = ln.split()
        if key == "case":
            cur = {"name": vals[0], "rows": []}
            cases.append(cur)
        elif key == "row":
            cur["rows"].append((int(vals[0]), vals[1], vals[2]))
        else:
            cur[key] = vals
    return cases


def _num(v):
    return float.fromhex(v) if "x" in v else float(v)


def _vecs(vals):
    return np.array([[_num(x) for x in v.split(",")] for v in vals])


def test_decode_attention_golden():
    cases = _attn_golden()
    assert [c["name"] for c in cases] == ["full", "window", "gqa"]
    for c in cases:
        n_q, n_kv = int(c["n_q"][0]), int(c["n_kv"][0])
        q = _vecs(c["q"])[None]                              # [1][n_q][d]
        d = q.shape[-1]
        n_rows = max(r for r, _, _ in c["rows"]) + 1
        kc = np.full((n_rows + 2, n_kv, d), 100.0)           # unlisted rows must not matter
        vc = np.full((n_rows + 2, n_kv, d), -100.0)
        for r, k, v in c["rows"]:
            kc[r] = _vecs(k.split(";"))
            vc[r] = _vecs(v.split(";"))
        out = attn.decode_attention(q, kc, vc, [int(c["base"][0])], [int(c["len"][0])], int(c["ring"][0]),
                                    int(c["window"][0]), [_num(s) for s in c["sinks"]], _num(c["scale"][0]))
        np.testing.assert_allclose(out[0], _vecs(c["out"]), rtol=1e-14, atol=1e-14, err_msg=c["name"])


def _random_cache(rng, n_rows, n_kv, d):
    return rng.standard_normal((n_rows, n_kv, d)), rng.standard_normal((n_rows, n_kv, d))


def test_decode_attention_without_sinks_is_textbook_attention():
    """Sinks at -inf: plain scaled dot-product attention over the attended
    rows, computed by torch's SDPA in float64 with the KV heads repeated
    for their query heads."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(11)
    n_q, n_kv, d, B = 8, 2, 16, 3
    kc, vc = _random_cache(rng, 200, n_kv, d)
    q = rng.standard_normal((B, n_q, d))
    base, lens, ring = [0, 60, 130], [7, 45, 60], 64
    scale = 1 / np.sqrt(d)
    out = attn.decode_attention(q, kc, vc, base, lens, ring, 0, np.full(n_q, -np.inf), scale)
    for b in range(B):
        rows = base[b] + np.arange(lens[b]) % ring
        k = torch.from_numpy(kc[rows]).permute(1, 0, 2).repeat_interleave(n_q // n_kv, 0)[None]
        v = torch.from_numpy(vc[rows]).permute(1, 0, 2).repeat_interleave(n_q // n_kv, 0)[None]
        want = F.scaled_dot_product_attention(torch.from_numpy(q[b])[None, :, None], k, v, scale=scale)
        np.testing.assert_allclose(out[b], want[0, :, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_decode_attention_sink_is_a_key_with_zero_value():
    """A sink acts as one more key whose score is the sink logit and whose
    value is zero: SDPA over the rows plus a zero key, with the sink added
    to that key's score by an additive mask."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(12)
    n_q, n_kv, d = 4, 4, 8
    kc, vc = _random_cache(rng, 32, n_kv, d)
    q = rng.standard_normal((1, n_q, d))
    sinks = rng.standard_normal(n_q) * 2
    scale = 0.3
    L, W = 20, 9
    out = attn.decode_attention(q, kc, vc, [5], [L], 27, W, sinks, scale)
    rows = 5 + np.arange(L - W, L) % 27
    k = np.concatenate([kc[rows], np.zeros((1, n_kv, d))]).transpose(1, 0, 2)
    v = np.concatenate([vc[rows], np.zeros((1, n_kv, d))]).transpose(1, 0, 2)
    mask = np.zeros((n_q, 1, W + 1))
    mask[:, 0, W] = sinks
    want = F.scaled_dot_product_attention(torch.from_numpy(q[0])[:, None], torch.from_numpy(k),
                                          torch.from_numpy(v), attn_mask=torch.from_numpy(mask), scale=scale)
    np.testing.assert_allclose(out[0], want[:, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_decode_attention_window_and_ring():
    """Only the window's rows matter (every other row can change freely),
    and a ring of C >= W rows gives the result of a contiguous layout."""
    rng = np.random.default_rng(13)
    n_q, n_kv, d, L, W = 4, 2, 8, 50, 13
    kc, vc = _random_cache(rng, L, n_kv, d)
    q = rng.standard_normal((1, n_q, d))
    sinks = rng.standard_normal(n_q)
    ref = attn.decode_attention(q, kc, vc, [0], [L], L, W, sinks, 0.5)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[: L - W] = rng.standard_normal(kc2[: L - W].shape) * 50
    vc2[: L - W] = 1e6
    np.testing.assert_array_equal(attn.decode_attention(q, kc2, vc2, [0], [L], L, W, sinks, 0.5), ref)
    for C in (W, W + 3, 64):
        kr = np.zeros((7 + C, n_kv, d))
        vr = np.zeros((7 + C, n_kv, d))
        for p in range(L - W, L):
            kr[7 + p % C], vr[7 + p % C] = kc[p], vc[p]
        np.testing.assert_allclose(attn.decode_attention(q, kr, vr, [7], [L], C, W, sinks, 0.5), ref,
                                   rtol=1e-14, atol=1e-15)
    # a window at least as long as the context is the full context
    np.testing.assert_array_equal(attn.decode_attention(q, kc, vc, [0], [L], L, L + 5, sinks, 0.5),
                                  attn.decode_attention(q, kc, vc, [0], [L], L, 0, sinks, 0.5))


def test_decode_attention_gqa_head_mapping():
    """Query head h reads KV head h // (n_q / n_kv): with a constant value
    row per KV head and no sink, head h returns KV head h // group's
    constant exactly."""
    rng = np.random.default_rng(14)
    n_q, n_kv, d = 12, 3, 8
    kc = rng.standard_normal((10, n_kv, d))
    vc = np.zeros((10, n_kv, d))
    for g in range(n_kv):
        vc[:, g, :] = float(g + 1)
    q = rng.standard_normal((2, n_q, d))
    out = attn.decode_attention(q, kc, vc, [0, 4], [4, 6], 6, 0, np.full(n_q, -np.inf), 1.0)
    for h in range(n_q):
        np.testing.assert_allclose(out[:, h], float(h // 4 + 1), rtol=1e-15)


def test_decode_attention_uniform_scores_closed_form():
    """Equal keys give equal scores s: out = mean(v) * L / (L + exp(sink - s));
    the |v| mixture equals the mixture itself for non-negative values."""
    rng = np.random.default_rng(15)
    n_q, n_kv, d, L = 2, 1, 8, 9
    kc = np.tile(rng.standard_normal(d), (L, n_kv, 1))
    vc = np.abs(rng.standard_normal((L, n_kv, d)))
    q = rng.standard_normal((1, n_q, d))
    sinks = np.array([0.7, -2.0])
    out, mix = attn.decode_attention(q, kc, vc, [0], [L], L, 0, sinks, 0.25, with_abs=True)
    for h in range(n_q):
        s = 0.25 * kc[0, 0] @ q[0, h]
        want = vc[:, 0].mean(axis=0) * L / (L + np.exp(sinks[h] - s))
        np.testing.assert_allclose(out[0, h], want, rtol=1e-13)
    np.testing.assert_array_equal(mix, out)
