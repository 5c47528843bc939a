"""Degenerate inputs through every decode path, the layer stack and prefill,
at the Flint shape (hidden 2048, 256 experts, top-6, shared expert):

  * an all-zero token: every logit is 0, so every score ties and the lowest
    indices 0..5 must be selected; the output is exactly zero;
  * an exact planted tie at the selection boundary: the router row of an
    expert ranked below 7th is replaced by the row of the 6th-ranked expert,
    so both logits are bit-identical on every path and the lower index must
    take the 6th place -- checked exactly (no near-tie exemption);
  * a NaN router row: its logit is NaN, which ranks below every number, so
    that expert is never selected;
  * a NaN scale byte (UE4M3 0x7F) in a selected expert: in a down row it
    makes exactly that output element NaN, in a gate row the whole token;
    NaN must appear exactly where the oracle has it.  In an unselected
    expert it changes nothing.

Ties by lower index and the NaN ordering are the readings of the method's
silent points (top-k of sigmoid scores, "Day-0 Support for Flint on vLLM",
"Model architecture"); NaN propagation follows from the UE4M3 decode.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gen
import w4a16_moe_decode_amd as fm
from _parity import check_routing, compare_outputs, compare_residual, oracle_experts, pack
from oracle import bf16 as obf
from oracle import moe

pytestmark = pytest.mark.gpu

SH = gen.SHAPE_FLINT
K = SH.top_k
NAN_BF16 = 0x7FC0
SCALE_POS = (0, 9, 18, 27)           # scale bytes of the interleaved super-block


@pytest.fixture(scope="module")
def base():
    return gen.moe_layer_source(SH, 900, "cpu")


def _with(src, *fields):
    """A copy of the layer source with the named tensors cloned (to edit)."""
    return dataclasses.replace(src, **{k: getattr(src, k).clone() for k in fields})


def _tokens(seed, n):
    return gen.activations(gen.seed_for(seed, "edge-x"), n, SH.hidden)


def _oracle_route(src, x):
    return moe.route(gen.numpy_f64(x), gen.numpy_f64(src.router), K, False)


def _plant_tie(src, x, lower: bool):
    """Copy the 6th-ranked expert's router row (for token x) into an expert
    ranked 9th or lower whose index is below (lower=True) or above it."""
    r = _oracle_route(src, x)
    order = np.argsort(-r.scores[0], kind="stable")
    b = int(order[K - 1])
    cands = [int(e) for e in order[K + 2:] if (e < b) == lower]
    a = cands[0]
    s = _with(src, "router")
    s.router[a] = s.router[b]
    return s, a, b


def _plant_nan_scale(src, expert, matrix, row):
    """UE4M3 NaN (0x7F) as the scale of columns 16..31 of `row` of the
    expert's `matrix` ("gate" or "down")."""
    s = _with(src, matrix)
    t = getattr(s, matrix)
    t[expert, row, 0, SCALE_POS[1]] = 0x7F
    return s


# ------------------------------------------------------------ decode paths --

PATHS = {"fused": (1, 0), "split": (1, fm.FLINT_SPLIT), "batch": (8, 0), "batch_split": (8, fm.FLINT_SPLIT)}
WANT_PATH = {"fused": fm.FLINT_PATH_SINGLE_ONE, "split": fm.FLINT_PATH_SPLIT,
             "batch": fm.FLINT_PATH_SINGLE_BATCH, "batch_split": fm.FLINT_PATH_SPLIT}


def _run_decode(src, x, path, renorm=False):
    batch, flags = PATHS[path]
    assert x.shape[0] == batch
    flags |= fm.FLINT_RENORM if renorm else 0
    layer = pack(src)
    runner = fm.DecodeRunner(layer, K, flags)
    assert fm.flint_moe_decode_path(runner.shape, batch) == WANT_PATH[path]
    idx = torch.full((batch, K), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((batch, K), dtype=torch.float32, device="cuda")
    out = runner(x.cuda(), topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    assert fm.decode_error_word(runner) == 0
    return gen.numpy_f64(out), idx.cpu().numpy(), w.cpu().numpy()


def _edge_batch(x_edge, path, seed):
    """The edge token alone (batch 1) or at position 3 of 8 tokens."""
    if PATHS[path][0] == 1:
        return x_edge, 0
    x = _tokens(seed, 8)
    x[3] = x_edge[0]
    return x, 3


def _oracle_out(src, x, idx_gpu, w_gpu, renorm=False):
    ex = oracle_experts(src)
    xo = gen.numpy_f64(x)
    _, r = moe.moe_layer(xo, ex, K, renorm)
    forced = check_routing(idx_gpu, w_gpu, r, renorm)
    want, _ = moe.moe_layer(xo, ex, K, renorm, forced_idx=forced)
    return want, r


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("renorm", [False, True])
def test_zero_token(base, path, renorm):
    x, t = _edge_batch(torch.zeros((1, SH.hidden), dtype=torch.bfloat16), path, 1)
    got, idx, w = _run_decode(base, x, path, renorm)
    assert list(idx[t]) == list(range(K))
    np.testing.assert_array_equal(w[t], np.full(K, 1.0 / K if renorm else 0.5, np.float32))
    assert np.all(got[t] == 0.0)
    want, _ = _oracle_out(base, x, idx, w, renorm)
    compare_outputs(got, want)


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("lower", [True, False])
def test_planted_tie_lower_index_wins(base, path, lower):
    xe = _tokens(2, 1)
    src, a, b = _plant_tie(base, xe, lower)
    x, t = _edge_batch(xe, path, 2)
    got, idx, w = _run_decode(src, x, path)
    r = _oracle_route(src, x)
    assert r.gap[t] == 0.0                      # the planted tie sits at the boundary
    win, lose = min(a, b), max(a, b)
    assert win in r.idx[t] and lose not in r.idx[t]
    assert list(idx[t]) == list(r.idx[t]), f"GPU {idx[t]} vs oracle {r.idx[t]} (tie {a}={b})"
    want, _ = _oracle_out(src, x, idx, w)
    compare_outputs(got, want)


@pytest.mark.parametrize("path", list(PATHS))
def test_nan_router_row_never_selected(base, path):
    xe = _tokens(3, 1)
    top = int(_oracle_route(base, xe).idx[0, 0])
    src = _with(base, "router")
    src.router[top] = torch.tensor(NAN_BF16, dtype=torch.int16).view(torch.bfloat16)
    x, t = _edge_batch(xe, path, 3)
    got, idx, w = _run_decode(src, x, path)
    assert not np.any(idx == top)
    want, r = _oracle_out(src, x, idx, w)
    assert top not in r.idx[t]
    compare_outputs(got, want)
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("matrix", ["down", "gate"])
def test_nan_scale_in_selected_expert(base, path, matrix):
    xe = _tokens(4, 1)
    e = int(_oracle_route(base, xe).idx[0, 2])
    row = 77
    src = _plant_nan_scale(base, e, matrix, row)
    x, t = _edge_batch(xe, path, 4)
    got, idx, w = _run_decode(src, x, path)
    assert e in idx[t]
    want, _ = _oracle_out(src, x, idx, w)
    if matrix == "down":
        assert np.isnan(want[t]).sum() == 1 and np.isnan(want[t, row])
    else:
        assert np.all(np.isnan(want[t]))
    compare_outputs(got, want)          # NaN exactly where the oracle has it


@pytest.mark.parametrize("path", list(PATHS))
def test_nan_scale_in_unselected_expert(base, path):
    xe = _tokens(5, 1)
    x, t = _edge_batch(xe, path, 5)
    sel = set(_oracle_route(base, x).idx.reshape(-1).tolist())
    e = next(i for i in range(SH.n_experts) if i not in sel)
    src = _plant_nan_scale(base, e, "down", 5)
    src = _plant_nan_scale(src, e, "gate", 6)
    got, idx, w = _run_decode(src, x, path)
    want, _ = _oracle_out(src, x, idx, w)
    assert np.all(np.isfinite(want))
    compare_outputs(got, want)


# ------------------------------------------------------------------ stack --

def _stack(srcs, gammas, x):
    dev = torch.device("cuda")
    layers = [pack(s) for s in srcs]
    step = fm.DecodeStep(layers, [g.to(dev) for g in gammas], [], [], K, stack=True)
    assert step.stack_shape is not None
    rec = []
    xd = x.to(dev)
    step(xd, record=rec)
    rec.append(xd.clone())
    torch.cuda.synchronize()
    assert fm.decode_error_word(step) == 0
    return step, [gen.numpy_f64(v) for v in rec]


def _check_stack_layers(step, srcs, gammas, rec):
    for l, src in enumerate(srcs):
        g = gen.numpy_f64(gammas[l])
        ex = oracle_experts(src)
        _, r = moe.moe_sublayer(rec[l], g, ex, K, False)
        idx, w = (v.cpu().numpy() for v in step.routing(l, 1))
        forced = check_routing(idx, w, r, False)
        want, _ = moe.moe_sublayer(rec[l], g, ex, K, False, forced_idx=forced)
        compare_residual(rec[l + 1], want, rec[l], f"stack layer {l}")
        yield l, idx, r


@pytest.fixture(scope="module")
def base2():
    return gen.moe_layer_source(SH, 901, "cpu")


def _gammas():
    return [gen.rmsnorm_gamma(gen.seed_for(9, "edge-g", l), SH.hidden) for l in range(2)]


def test_stack_zero_token(base, base2):
    gm = _gammas()
    step, rec = _stack([base, base2], gm, torch.zeros((1, SH.hidden), dtype=torch.bfloat16))
    for l, idx, _ in _check_stack_layers(step, [base, base2], gm, rec):
        assert list(idx[0]) == list(range(K)), f"layer {l}"
    assert np.all(rec[-1] == 0.0)


@pytest.mark.parametrize("lower", [True, False])
def test_stack_planted_tie(base, base2, lower):
    gm = _gammas()
    x = _tokens(6, 1)
    xn = obf.round_bf16(moe.rmsnorm(gen.numpy_f64(x), gen.numpy_f64(gm[0])))
    src0, a, b = _plant_tie(base, torch.tensor(xn, dtype=torch.float32).to(torch.bfloat16), lower)
    step, rec = _stack([src0, base2], gm, x)
    for l, idx, r in _check_stack_layers(step, [src0, base2], gm, rec):
        if l == 0:
            assert r.gap[0] == 0.0
            assert list(idx[0]) == list(r.idx[0]) and min(a, b) in idx[0] and max(a, b) not in idx[0]


def test_stack_nan_scale_last_layer(base, base2):
    gm = _gammas()
    x = _tokens(7, 1)
    step, _ = _stack([base, base2], gm, x)
    e = int(step.routing(1, 1)[0][0, 1].item())       # an expert layer 1 selects
    src1 = _plant_nan_scale(base2, e, "down", 300)
    step, rec = _stack([base, src1], gm, x)
    assert e in step.routing(1, 1)[0].cpu().numpy()
    list(_check_stack_layers(step, [base, src1], gm, rec))
    assert np.isnan(rec[-1]).sum() == 1 and np.isnan(rec[-1][0, 300])


# ---------------------------------------------------------------- prefill --

def _run_prefill(src, x):
    layer = pack(src)
    T = x.shape[0]
    runner = fm.PrefillRunner(layer, K, T, 0)
    idx = torch.full((T, K), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((T, K), dtype=torch.float32, device="cuda")
    out = runner(x.cuda(), topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    return gen.numpy_f64(out), idx.cpu().numpy(), w.cpu().numpy()


def test_prefill_zero_token(base):
    x = _tokens(10, 8)
    x[5] = 0
    got, idx, w = _run_prefill(base, x)
    assert list(idx[5]) == list(range(K)) and np.all(got[5] == 0.0)
    want, _ = _oracle_out(base, x, idx, w)
    compare_outputs(got, want)


@pytest.mark.parametrize("lower", [True, False])
def test_prefill_planted_tie(base, lower):
    x = _tokens(11, 8)
    src, a, b = _plant_tie(base, x[2:3], lower)
    got, idx, w = _run_prefill(src, x)
    r = _oracle_route(src, x)
    assert r.gap[2] == 0.0
    assert list(idx[2]) == list(r.idx[2]) and min(a, b) in idx[2] and max(a, b) not in idx[2]
    want, _ = _oracle_out(src, x, idx, w)
    compare_outputs(got, want)


def test_prefill_nan_router_row_and_nan_scales(base):
    x = _tokens(12, 8)
    r = _oracle_route(base, x)
    top = int(r.idx[0, 0])
    src = _with(base, "router")
    src.router[top] = torch.tensor(NAN_BF16, dtype=torch.int16).view(torch.bfloat16)
    r2 = _oracle_route(src, x)
    e = int(r2.idx[4, 1])
    src = _plant_nan_scale(src, e, "down", 1000)
    got, idx, w = _run_prefill(src, x)
    assert not np.any(idx == top)
    want, _ = _oracle_out(src, x, idx, w)
    hit = [t for t in range(8) if e in idx[t]]
    assert 4 in hit
    for t in range(8):
        assert np.isnan(want[t]).sum() == (1 if t in hit else 0)
    compare_outputs(got, want)
