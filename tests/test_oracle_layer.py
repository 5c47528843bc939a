"""Pins of the oracle's layer arithmetic (CPU only).

Each test ties a piece of the oracle to an independent statement: a
brute-force definition, a library routine, a closed form on a special
input, or an invariant the method implies (unselected experts contribute
nothing, the shared expert is always added, prefill equals per-token decode).
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import gen
from oracle import bf16, formats, moe

SH = gen.SHAPE_TINY


def _bf(a):
    return torch.tensor(a, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).numpy()


def _experts_from_source(src, layout="interleaved"):
    u8 = gen.numpy_u8
    return moe.nvfp4_expert_set(
        gen.numpy_f64(src.router), u8(src.gate), u8(src.up), u8(src.down), src.gscale.numpy(),
        None if src.sh_gate is None else u8(src.sh_gate),
        None if src.sh_up is None else u8(src.sh_up),
        None if src.sh_down is None else u8(src.sh_down), src.sh_gscale.numpy(), layout)


# ------------------------------------------------------------- top-k ------

def _rank_count_topk(s, k):
    """Brute force: expert i beats j when s_i > s_j, or equal and i < j;
    i is selected when fewer than k experts beat it, placed at that rank."""
    n = len(s)
    rank = [sum(1 for j in range(n) if s[j] > s[i] or (s[j] == s[i] and j < i)) for i in range(n)]
    out = [None] * k
    for i in range(n):
        if rank[i] < k:
            out[rank[i]] = i
    return out


@pytest.mark.parametrize("seed", range(8))
def test_topk_matches_rank_count_bruteforce(seed):
    rng = np.random.default_rng(seed)
    n, k = (32, 4) if seed % 2 else (256, 6)
    s = rng.random(n)
    # plant ties, including across the selection boundary
    s[rng.integers(0, n, 6)] = s[np.argsort(-s)[k - 1]]
    s[rng.integers(0, n, 3)] = s[np.argsort(-s)[0]]
    idx, gap = moe.topk_select(s, k)
    assert list(idx) == _rank_count_topk(list(s), k)
    srt = sorted(s, reverse=True)
    assert gap == srt[k - 1] - srt[k]


@pytest.mark.parametrize("seed", range(4))
def test_topk_nan_score_ranks_lowest(seed):
    """A NaN score is never selected while k numbers remain: the selection
    equals the top-k of the scores with the NaN entries taken out."""
    rng = np.random.default_rng(100 + seed)
    n, k = 256, 6
    s = rng.random(n)
    bad = rng.choice(n, 3, replace=False)
    bad[0] = int(np.argmax(s))                     # the largest score becomes NaN
    s[bad] = np.nan
    keep = np.array([i for i in range(n) if i not in set(bad.tolist())])
    idx, gap = moe.topk_select(s, k)
    sub, sub_gap = moe.topk_select(s[keep], k)
    assert list(idx) == list(keep[sub]) and gap == sub_gap
    assert not set(idx.tolist()) & set(bad.tolist())


def test_zero_input_ties_select_lowest_indices():
    src = gen.moe_layer_source(SH, 5)
    ex = _experts_from_source(src)
    r = moe.route(np.zeros((1, SH.hidden)), ex.router, SH.top_k, renorm=False)
    assert list(r.idx[0]) == list(range(SH.top_k))
    np.testing.assert_array_equal(r.weight[0], 0.5)
    assert r.gap[0] == 0.0
    rn = moe.route(np.zeros((1, SH.hidden)), ex.router, SH.top_k, renorm=True)
    np.testing.assert_array_equal(rn.weight[0], 1.0 / SH.top_k)


def test_renorm_weights_sum_to_one_and_scale_raw():
    src = gen.moe_layer_source(SH, 6)
    ex = _experts_from_source(src)
    x = gen.numpy_f64(gen.activations(7, 4, SH.hidden))
    raw = moe.route(x, ex.router, SH.top_k, renorm=False)
    ren = moe.route(x, ex.router, SH.top_k, renorm=True)
    np.testing.assert_array_equal(raw.idx, ren.idx)
    np.testing.assert_allclose(ren.weight.sum(1), 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(ren.weight * raw.weight.sum(1, keepdims=True), raw.weight, rtol=1e-15)
    # raw weights are the sigmoid of the router logits (library sigmoid)
    lib = torch.sigmoid(torch.tensor(raw.logits)).numpy()
    np.testing.assert_allclose(raw.weight, np.take_along_axis(lib, raw.idx, 1), rtol=1e-15)


# ------------------------------------------------------ elementwise pieces --

def test_silu_matches_torch():
    z = np.linspace(-30, 30, 10001)
    np.testing.assert_allclose(moe.silu(z), F.silu(torch.tensor(z)).numpy(), rtol=1e-14, atol=1e-300)


def test_rmsnorm_matches_torch_rms_norm_then_rounds():
    rng = np.random.default_rng(2)
    x = _bf(rng.standard_normal((3, 512)))
    gamma = _bf(1 + 0.1 * rng.standard_normal(512))
    lib = F.rms_norm(torch.tensor(x), (512,), eps=1e-6).numpy()
    want = bf16.round_bf16(bf16.round_bf16(lib) * gamma)
    got = moe.rmsnorm(x, gamma, 1e-6)
    # library and oracle may differ in the last float64 bit before rounding
    assert np.mean(got == want) > 0.999
    np.testing.assert_allclose(got, want, rtol=2 ** -7)
    # constant input: x / rms(x) = sign(x) up to eps, so xn = gamma
    c = np.full((1, 512), 3.0)
    np.testing.assert_array_equal(moe.rmsnorm(c, gamma, 1e-6)[0], gamma)


def test_rmsnorm_golden_small_mean_square():
    """mean(x^2) of the order of eps: where eps sits decides the result
    (hand-derived rows in tests/golden/rmsnorm_small_ms.txt)."""
    path = os.path.join(os.path.dirname(__file__), "golden", "rmsnorm_small_ms.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 2
    for _, xs, gs, want in rows:
        x = np.array([float.fromhex(v) for v in xs.split(",")])[None, :]
        gamma = np.array([float(v) for v in gs.split(",")])
        got = moe.rmsnorm(x, gamma, 1e-6)[0]
        np.testing.assert_array_equal(got, np.array([float(v) for v in want.split(",")]))


# ------------------------------------------------------- expert structure --

def test_expert_ffn_orientation_one_hot():
    """One-hot input picks column j of W_gate/W_up; a gate with one live row
    picks column i of W_down: catches any transposed operand."""
    rng = np.random.default_rng(4)
    H, I = 64, 128
    wg = np.zeros((I, H))
    wu = _bf(rng.standard_normal((I, H)))
    wd = _bf(rng.standard_normal((H, I)))
    i, j = 37, 11
    wg[i, j] = 2.0
    z = np.zeros(H)
    z[j] = 1.0
    y, (g, u, h) = moe.expert_ffn(z, wg, wu, wd)
    np.testing.assert_array_equal(g, wg[:, j])
    np.testing.assert_array_equal(u, wu[:, j])
    a = _bf(2.0 / (1.0 + math.exp(-2.0)))                 # SiLU(2) rounded
    hi = _bf(a * u[i])
    assert np.count_nonzero(h) == (1 if hi != 0 else 0) and h[i] == hi
    np.testing.assert_array_equal(y, wd[:, i] * hi)


def _const_blocks(n, rows, cols, code_byte, scale_byte, layout="interleaved"):
    """Source blocks whose every value is E2M1(code nibble) * UE4M3(scale)."""
    b = np.full((n, rows, cols // 64, 36), code_byte, np.uint8)
    pos = [0, 9, 18, 27] if layout == "interleaved" else [0, 1, 2, 3]
    b[..., pos] = scale_byte
    return b


def test_layer_closed_form_constant_experts():
    """Constant matrices reduce every GEMV to a scalar: the layer output can
    be written down by hand for this input."""
    H, I, E, K = 64, 64, 4, 2
    c = [0.5, 1.0, -1.0, 0.25]                        # router logit of expert e when x = 1
    router = np.repeat(np.array(c)[:, None] / 64, H, 1)   # c_e / 64 is exact in bf16
    # gate/up/down values: code byte 0x22 -> both nibbles 1.0; scale byte picks the value
    gate = np.stack([_const_blocks(1, I, H, 0x22, sb)[0] for sb in (0x38, 0x30, 0x40, 0x38)])
    up = np.stack([_const_blocks(1, I, H, 0x22, sb)[0] for sb in (0x30, 0x38, 0x38, 0x40)])
    down = np.stack([_const_blocks(1, H, I, 0x22, sb)[0] for sb in (0x38, 0x40, 0x30, 0x38)])
    gs = np.array([[1 / 64, 1 / 64, 1 / 64]] * E)
    shg = _const_blocks(1, I, H, 0x22, 0x38)
    shu = _const_blocks(1, I, H, 0x22, 0x38)
    shd = _const_blocks(1, H, I, 0x22, 0x30)
    ex = moe.nvfp4_expert_set(router, gate, up, down, gs, shg, shu, shd, np.array([1 / 64] * 3))
    x = np.ones((1, H))
    out, r = moe.moe_layer(x, ex, K, renorm=False)
    # expected: experts 1 and 0 win (logits 1.0 and 0.5)
    assert list(r.idx[0]) == [1, 0]
    sig = lambda v: 1 / (1 + math.exp(-v))
    # per expert e: every weight of a matrix = scale value / 64; over 64 inputs
    # of 1 the gate/up dot products equal the scale values
    sv = {0x38: 1.0, 0x30: 0.5, 0x40: 2.0}
    gate_v = [1.0, 0.5, 2.0, 1.0]
    up_v = [0.5, 1.0, 1.0, 2.0]
    down_v = [1.0, 2.0, 0.5, 1.0]

    def expert_out(gv, uv, dv):
        hval = _bf(_bf(gv * sig(gv)) * uv)        # h, identical in all I rows
        return I * (dv / 64) * hval                # each output row sums I equal terms

    acc = (sig(1.0) * expert_out(gate_v[1], up_v[1], down_v[1])
           + sig(0.5) * expert_out(gate_v[0], up_v[0], down_v[0])
           + expert_out(1.0, 1.0, sv[0x30]))
    np.testing.assert_array_equal(out[0], np.full(H, _bf(acc)))


def test_unselected_experts_contribute_nothing():
    """Computing every expert and weighting the unselected ones by zero gives
    the same output as reading only the selected experts."""
    src = gen.moe_layer_source(SH, 8)
    ex = _experts_from_source(src)
    x = gen.numpy_f64(gen.activations(9, 3, SH.hidden))
    out, r = moe.moe_layer(x, ex, SH.top_k, renorm=True)
    for t in range(3):
        wfull = np.zeros(SH.n_experts)
        wfull[r.idx[t]] = r.weight[t]
        acc = sum(wfull[e] * moe.expert_ffn(x[t], *ex.expert(e))[0] for e in range(SH.n_experts))
        acc = acc + moe.expert_ffn(x[t], *ex.expert(None))[0]
        dense = bf16.round_bf16(acc)
        ulp = np.abs(dense) * 2 ** -7 + 1e-30
        assert np.all(np.abs(dense - out[t]) <= ulp)
        assert np.mean(dense == out[t]) > 0.99


def test_shared_expert_always_added():
    src = gen.moe_layer_source(SH, 10)
    x = gen.numpy_f64(gen.activations(11, 2, SH.hidden))
    # zero every routed code: routed experts give exactly zero
    z = gen.moe_layer_source(SH, 10)
    for t in (z.gate, z.up, z.down):
        keep = t[..., [0, 9, 18, 27]].clone()
        t.zero_()
        t[..., [0, 9, 18, 27]] = keep
    ex0 = _experts_from_source(z)
    out, _ = moe.moe_layer(x, ex0, SH.top_k, renorm=False)
    wg, wu, wd = ex0.expert(None)
    np.testing.assert_array_equal(out, moe.dense_mlp(x, wg, wu, wd))
    # zero the shared expert instead: output is the routed part alone
    ex = _experts_from_source(src)
    s2 = gen.moe_layer_source(SH, 10)
    s2.sh_down.zero_()
    ex2 = _experts_from_source(s2)
    out2, r = moe.moe_layer(x, ex2, SH.top_k, renorm=False)
    for t in range(2):
        acc = sum(r.weight[t, k] * moe.expert_ffn(x[t], *ex.expert(int(r.idx[t, k])))[0]
                  for k in range(SH.top_k))
        np.testing.assert_array_equal(out2[t], bf16.round_bf16(acc))
    # no shared expert at all (shared_inter = 0)
    s3 = gen.moe_layer_source(gen.MoeShape(SH.hidden, SH.n_experts, SH.inter, 0, SH.top_k), 10)
    out3, _ = moe.moe_layer(x, _experts_from_source(s3), SH.top_k, renorm=False)
    np.testing.assert_array_equal(out3, out2)


def test_tensor_scale_multiplies_exactly():
    src = gen.moe_layer_source(SH, 12)
    ex1 = _experts_from_source(src)
    src.gscale[:, 0] *= 2.0     # gate scale doubled: g doubles exactly
    ex2 = _experts_from_source(src)
    z = gen.numpy_f64(gen.activations(13, 1, SH.hidden))[0]
    _, (g1, u1, _) = moe.expert_ffn(z, *ex1.expert(3))
    _, (g2, u2, _) = moe.expert_ffn(z, *ex2.expert(3))
    np.testing.assert_array_equal(g2, 2 * g1)
    np.testing.assert_array_equal(u2, u1)


def test_prefill_equals_per_token_decode_and_histogram():
    src = gen.moe_layer_source(SH, 14)
    ex = _experts_from_source(src)
    x = gen.numpy_f64(gen.activations(15, 6, SH.hidden))
    out, r = moe.prefill(x, ex, SH.top_k, renorm=False)
    for t in range(6):
        o1, r1 = moe.moe_layer(x[t:t + 1], ex, SH.top_k, renorm=False)
        np.testing.assert_array_equal(out[t], o1[0])
        np.testing.assert_array_equal(r.idx[t], r1.idx[0])
    h = moe.expert_histogram(r.idx, SH.n_experts)
    assert h.sum() == 6 * SH.top_k and h.shape == (SH.n_experts,)
    sub, _ = moe.prefill(x, ex, SH.top_k, renorm=False, tokens=[4, 1])
    np.testing.assert_array_equal(sub, out[[4, 1]])


def test_sublayers_add_residual_once_rounded():
    src = gen.moe_layer_source(SH, 16)
    ex = _experts_from_source(src)
    x = gen.numpy_f64(gen.activations(17, 2, SH.hidden))
    gamma = gen.numpy_f64(gen.rmsnorm_gamma(18, SH.hidden))
    xn = moe.rmsnorm(x, gamma)
    out, _ = moe.moe_layer(xn, ex, SH.top_k, renorm=True)
    new, _ = moe.moe_sublayer(x, gamma, ex, SH.top_k, renorm=True)
    np.testing.assert_array_equal(new, bf16.round_bf16(x + out))
    wg, wu, wd = ex.expert(None)
    dn = moe.dense_sublayer(x, gamma, wg, wu, wd)
    np.testing.assert_array_equal(dn, bf16.round_bf16(x + moe.dense_mlp(xn, wg, wu, wd)))


def test_forced_idx_overrides_selection():
    src = gen.moe_layer_source(SH, 19)
    ex = _experts_from_source(src)
    x = gen.numpy_f64(gen.activations(20, 1, SH.hidden))
    forced = [[5, 9, 2, 30]]
    out, r = moe.moe_layer(x, ex, SH.top_k, renorm=False, forced_idx=forced)
    assert list(r.idx[0]) == forced[0]
    np.testing.assert_array_equal(r.weight[0], r.scores[0, forced[0]])


def test_generator_statistics():
    """The input recipe: E[w^2] of the NVFP4 weights, router logit spread."""
    src = gen.moe_layer_source(gen.SHAPE_FLINT, 0)
    w = formats.decode_source_matrix(gen.numpy_u8(src.gate[0]), "interleaved", 1 / 64)
    assert abs(np.mean(w ** 2) - 0.00637) < 0.0002
    x = gen.numpy_f64(gen.activations(1, 8, 2048))
    logits = x @ gen.numpy_f64(src.router).T
    assert 0.85 < np.std(logits) < 0.96
    a = gen.nvfp4_source(1, 1, 4, 128)
    b = gen.nvfp4_source(1, 1, 4, 128)
    assert torch.equal(a, b)
    assert set(np.unique(gen.numpy_u8(a)[..., [0, 9, 18, 27]])) <= {e << 3 for e in range(3, 10)}
