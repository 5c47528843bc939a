"""The single-launch batch-1 decode path (hidden 2048 or 4096, NVFP4)
against the oracle and against the three-kernel path (FLINT_SPLIT)."""
import pytest
import torch

import gen
import w4a16_moe_decode_amd as fm
from _parity import DecodeCase, compare_outputs, pack, run_decode_case

pytestmark = pytest.mark.gpu

FLINT = gen.SHAPE_FLINT


@pytest.mark.parametrize("shape", [
    FLINT,
    gen.MoeShape(hidden=4096, n_experts=64, inter=256, shared_inter=512, top_k=6),    # 2 chunks per lane
    gen.MoeShape(hidden=2048, n_experts=48, inter=512, shared_inter=1024, top_k=8),   # wide shared, K=8
    gen.MoeShape(hidden=2048, n_experts=300 // 2, inter=128, shared_inter=0, top_k=4),  # no shared
    gen.MoeShape(hidden=2048, n_experts=16, inter=2048, shared_inter=64, top_k=2),    # widest routed
], ids=["flint", "h4096", "wide-shared-k8", "no-shared", "wide-routed"])
@pytest.mark.parametrize("flags", [0, fm.FLINT_RENORM, fm.FLINT_PRE_RMSNORM | fm.FLINT_RESIDUAL])
def test_fused_against_oracle(shape, flags):
    src = gen.moe_layer_source(shape, 500 + shape.hidden + shape.n_experts)
    layer = pack(src)
    for seed in (1, 2):
        run_decode_case(DecodeCase(shape, seed=seed, batch=1, flags=flags), src=src, layer=layer)


def test_fused_matches_split_and_is_reproducible():
    src = gen.moe_layer_source(FLINT, 600)
    layer = pack(src)
    fused = fm.DecodeRunner(layer, FLINT.top_k, 0)
    split = fm.DecodeRunner(layer, FLINT.top_k, fm.FLINT_SPLIT)
    for i in range(4):
        x = gen.activations(700 + i, 1, FLINT.hidden).cuda()
        a = fused(x)
        b = fused(x)
        c = split(x)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        compare_outputs(a.cpu().float().numpy(), c.cpu().float().numpy(), "fused vs split")


def test_fused_and_split_share_a_workspace():
    """Batch-1 (single launch) and batch-8 (three kernels) calls alternate on
    one workspace; the launch epoch keeps their hand-off words apart."""
    src = gen.moe_layer_source(FLINT, 601)
    layer = pack(src)
    r = fm.DecodeRunner(layer, FLINT.top_k, 0)
    for i, b in enumerate([1, 8, 1, 1, 3, 1]):
        run_decode_case(DecodeCase(FLINT, seed=800 + i, batch=b), src=src, layer=layer, runner=r)
    assert fm.decode_error_word(r) == 0


def test_fused_error_word_stays_clear():
    src = gen.moe_layer_source(FLINT, 602)
    layer = pack(src)
    r = fm.DecodeRunner(layer, FLINT.top_k, 0)
    x = gen.activations(9, 1, FLINT.hidden).cuda()
    for _ in range(20):
        r(x)
    torch.cuda.synchronize()
    assert fm.decode_error_word(r) == 0
