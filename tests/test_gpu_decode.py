"""Decode MoE layer on the GPU (through flint_moe_decode) against the oracle.

Cases span the tiny and Flint-shaped layers, batch 1..8, both combine
modes, both source byte orders, every UE4M3 mantissa, non-power-of-two
tensor scales, ragged shapes (row tiles with tails, lane groups with idle
lanes), no shared expert, a shared expert of another width, the all-tie
zero input, pre-norm + residual, and BF16 weights."""
import dataclasses

import numpy as np
import pytest
import torch

import gen
import w4a16_moe_decode_amd as fm
from _parity import DecodeCase, compare_outputs, pack, run_decode_case
from oracle import moe

pytestmark = pytest.mark.gpu

TINY = gen.SHAPE_TINY
FLINT = gen.SHAPE_FLINT


@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("batch", [1, 2, 5, 8])
def test_tiny_layer(batch, renorm):
    run_decode_case(DecodeCase(TINY, seed=11, batch=batch, flags=fm.FLINT_RENORM if renorm else 0))


@pytest.mark.parametrize("case", [
    DecodeCase(TINY, seed=3, batch=3, layout="scales_first"),
    DecodeCase(TINY, seed=4, batch=4, scale_mode="full"),
    DecodeCase(TINY, seed=5, batch=2, gscale_mode="varied", flags=fm.FLINT_RENORM),
    DecodeCase(TINY, seed=6, batch=8, x_kind="correlated"),
    DecodeCase(TINY, seed=7, batch=1, zero_x=True),
    DecodeCase(TINY, seed=8, batch=6, flags=fm.FLINT_PRE_RMSNORM | fm.FLINT_RESIDUAL),
    DecodeCase(TINY, seed=9, batch=3, wbf16=True),
    DecodeCase(TINY, seed=9, batch=1, wbf16=True, flags=fm.FLINT_RENORM),
], ids=lambda c: f"b{c.batch}-{c.layout}-{c.scale_mode}-{c.gscale_mode}-{c.x_kind}-z{int(c.zero_x)}-f{c.flags}-bf{int(c.wbf16)}")
def test_tiny_layer_variants(case):
    run_decode_case(case)


@pytest.mark.parametrize("shape,batch", [
    (gen.MoeShape(hidden=576, n_experts=40, inter=192, shared_inter=320, top_k=5), 3),  # ragged
    (gen.MoeShape(hidden=64, n_experts=1, inter=64, shared_inter=64, top_k=1), 2),      # minimum
    (gen.MoeShape(hidden=256, n_experts=16, inter=64, shared_inter=0, top_k=8), 8),     # no shared, K=8
    (gen.MoeShape(hidden=1088, n_experts=256, inter=128, shared_inter=128, top_k=6), 7),
    (gen.MoeShape(hidden=3072, n_experts=64, inter=128, shared_inter=256, top_k=4), 3),  # widest hidden
])
def test_ragged_and_edge_shapes(shape, batch):
    run_decode_case(DecodeCase(shape, seed=21, batch=batch))
    run_decode_case(DecodeCase(shape, seed=22, batch=batch, wbf16=True, flags=fm.FLINT_RENORM))


def abi(sh, flags):
    return fm.FlintMoeShape(sh.hidden, sh.n_experts, sh.inter, sh.shared_inter, sh.top_k, flags, 1e-6)


@pytest.fixture(scope="module")
def flint_layer():
    src = gen.moe_layer_source(FLINT, 100, "cpu")
    layer = pack(src)
    return src, layer


@pytest.mark.parametrize("batch,flags", [
    (1, 0), (1, fm.FLINT_RENORM), (8, 0), (8, fm.FLINT_RENORM), (4, 0), (2, 0), (3, fm.FLINT_RENORM),
    (5, 0), (7, fm.FLINT_RENORM), (8, fm.FLINT_PRE_RMSNORM | fm.FLINT_RESIDUAL),
    (3, fm.FLINT_PRE_RMSNORM | fm.FLINT_RESIDUAL | fm.FLINT_RENORM),
    (8, fm.FLINT_SPLIT), (5, fm.FLINT_SPLIT | fm.FLINT_RENORM),
    (8, fm.FLINT_SPLIT | fm.FLINT_PRE_RMSNORM | fm.FLINT_RESIDUAL),
])
def test_flint_layer(flint_layer, batch, flags):
    """Batch 1 runs as one launch, batch 2..8 as the batch single launch,
    FLINT_SPLIT as three kernels."""
    src, layer = flint_layer
    want = (fm.FLINT_PATH_SPLIT if flags & fm.FLINT_SPLIT else
            fm.FLINT_PATH_SINGLE_ONE if batch == 1 else fm.FLINT_PATH_SINGLE_BATCH)
    assert fm.flint_moe_decode_path(abi(FLINT, flags), batch) == want
    run_decode_case(DecodeCase(FLINT, seed=100 + batch + flags, batch=batch, flags=flags),
                    src=src, layer=layer)


@pytest.mark.parametrize("top_k,batch", [(8, 8), (8, 3), (1, 8), (2, 2), (6, 8)])
def test_flint_batch_top_k(top_k, batch):
    """The batch single launch with a top-k other than the usual 6 (its
    general variant) and with 6 against a fresh layer: up to 64 routed slots
    at k = 8, one routed expert per token at k = 1."""
    sh = dataclasses.replace(FLINT, top_k=top_k)
    assert fm.flint_moe_decode_path(abi(sh, 0), batch) == fm.FLINT_PATH_SINGLE_BATCH
    src = gen.moe_layer_source(sh, 150 + top_k, "cpu")
    layer = pack(src)
    for flags in (0, fm.FLINT_RENORM):
        run_decode_case(DecodeCase(sh, seed=160 + top_k + batch + flags, batch=batch, flags=flags),
                        src=src, layer=layer)


@pytest.mark.parametrize("top_k", [1, 8])
def test_flint_layer_bf16_weights_top_k(top_k):
    """The BF16 form of the batch-1 single launch with a top-k other than 6
    (its general variant): one routed expert, and eight (slot 8 on wave 7)."""
    sh = dataclasses.replace(FLINT, top_k=top_k)
    assert fm.flint_moe_decode_path(abi(sh, fm.FLINT_W_BF16), 1) == fm.FLINT_PATH_SINGLE_ONE
    src = gen.moe_layer_source(sh, 170 + top_k, "cpu")
    layer = pack(src)
    layer.add_bf16()
    for flags in (0, fm.FLINT_RENORM | fm.FLINT_PRE_RMSNORM | fm.FLINT_RESIDUAL):
        run_decode_case(DecodeCase(sh, seed=180 + top_k + flags, batch=1, wbf16=True, flags=flags),
                        src=src, layer=layer)


def test_flint_layer_bf16_weights(flint_layer):
    """W16A16 at the Flint shape: batch 1 runs the BF16 form of the single
    launch (also with pre-norm + residual and renormalised weights), batch 8
    the three kernels."""
    src, layer = flint_layer
    layer.add_bf16()
    try:
        assert fm.flint_moe_decode_path(abi(FLINT, fm.FLINT_W_BF16), 1) == fm.FLINT_PATH_SINGLE_ONE
        run_decode_case(DecodeCase(FLINT, seed=200, batch=1, wbf16=True), src=src, layer=layer)
        run_decode_case(DecodeCase(FLINT, seed=202, batch=1, wbf16=True, flags=fm.FLINT_RENORM), src=src, layer=layer)
        run_decode_case(DecodeCase(FLINT, seed=203, batch=1, wbf16=True,
                                   flags=fm.FLINT_PRE_RMSNORM | fm.FLINT_RESIDUAL), src=src, layer=layer)
        run_decode_case(DecodeCase(FLINT, seed=201, batch=8, wbf16=True), src=src, layer=layer)
    finally:
        layer.gu_bf16 = layer.d_bf16 = layer.sh_gu_bf16 = layer.sh_d_bf16 = None


def test_zero_input_routes_to_lowest_experts(flint_layer):
    src, layer = flint_layer
    _, _, r = run_decode_case(DecodeCase(FLINT, seed=300, batch=2, zero_x=True), src=src, layer=layer)
    assert list(r.idx[0]) == list(range(6))


def test_results_are_bit_reproducible_and_stages_compose(flint_layer):
    """No float atomics: two runs give identical bits, on the single-launch
    path and on the three-kernel one; running the three stages by hand equals
    one three-kernel call."""
    _, layer = flint_layer
    runner = fm.DecodeRunner(layer, FLINT.top_k, 0)
    split = fm.DecodeRunner(layer, FLINT.top_k, fm.FLINT_SPLIT)
    assert fm.flint_moe_decode_path(runner.shape, 1) == fm.FLINT_PATH_SINGLE_ONE
    x = gen.activations(7, 1, FLINT.hidden).cuda()
    a = runner(x)
    b = runner(x)
    s1 = split(x)
    s2 = split(x)
    c = torch.empty_like(x)
    for st in range(3):
        split.stage(st, x, c)
    x8 = gen.activations(8, 8, FLINT.hidden).cuda()
    d1 = runner(x8)
    d2 = runner(x8)
    e1 = split(x8)
    e2 = split(x8)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(s1, s2) and torch.equal(s1, c)
    assert torch.equal(d1, d2) and torch.equal(e1, e2)
    compare_outputs(d1.cpu().float().numpy(), e1.cpu().float().numpy(), "batch single launch vs split")


def test_rotating_copies_and_workspace_reuse(flint_layer):
    """One workspace serves consecutive calls of different batch sizes and
    layers."""
    src, layer = flint_layer
    src2 = gen.moe_layer_source(FLINT, 101, "cpu")
    layer2 = pack(src2)
    r1 = fm.DecodeRunner(layer, FLINT.top_k, 0)
    r2 = fm.DecodeRunner(layer2, FLINT.top_k, 0)
    r2.ws = r1.ws
    for i, bsz in enumerate([8, 1, 3, 8, 2]):
        s, L, R = (src, layer, r1) if i % 2 == 0 else (src2, layer2, r2)
        run_decode_case(DecodeCase(FLINT, seed=400 + i, batch=bsz), src=s, layer=L, runner=R)
