"""The single-launch decode path (batch 1; hidden 2048 or 4096, NVFP4)
against the oracle and against the three-kernel path (FLINT_SPLIT)."""
import pytest
import torch

import gen
import w4a16_moe_decode_amd as fm
from _parity import DecodeCase, compare_outputs, pack, run_decode_case

pytestmark = pytest.mark.gpu

FLINT = gen.SHAPE_FLINT


SHAPES = [
    FLINT,
    gen.MoeShape(hidden=4096, n_experts=64, inter=256, shared_inter=512, top_k=6),    # 2 chunks per lane
    gen.MoeShape(hidden=2048, n_experts=48, inter=512, shared_inter=1024, top_k=8),   # wide shared, K=8
    gen.MoeShape(hidden=2048, n_experts=300 // 2, inter=128, shared_inter=0, top_k=4),  # no shared
    gen.MoeShape(hidden=2048, n_experts=16, inter=2048, shared_inter=64, top_k=2),    # widest routed
]
SHAPE_IDS = ["flint", "h4096", "wide-shared-k8", "no-shared", "wide-routed"]
FLAG_SETS = [0, fm.FLINT_RENORM, fm.FLINT_PRE_RMSNORM | fm.FLINT_RESIDUAL]


@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
@pytest.mark.parametrize("flags", FLAG_SETS)
def test_fused_against_oracle(shape, flags):
    src = gen.moe_layer_source(shape, 500 + shape.hidden + shape.n_experts)
    layer = pack(src)
    r = fm.DecodeRunner(layer, shape.top_k, flags)
    # the widest routed expert needs more down-row items than the one-token
    # kernel keeps in flight (3 slots x 8 chunk steps > 20): three kernels
    want = fm.FLINT_PATH_SPLIT if shape.inter == 2048 else fm.FLINT_PATH_SINGLE_ONE
    assert fm.flint_moe_decode_path(r.shape, 1) == want
    for seed in (1, 2):
        run_decode_case(DecodeCase(shape, seed=seed, batch=1, flags=flags), src=src, layer=layer,
                        runner=r)


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
    """Batch-1 single launches and three-kernel calls (batch 1 with
    FLINT_SPLIT, batches 2..8) alternate on one workspace; the launch epoch
    keeps their hand-off words apart."""
    src = gen.moe_layer_source(FLINT, 601)
    layer = pack(src)
    r = fm.DecodeRunner(layer, FLINT.top_k, 0)
    s = fm.DecodeRunner(layer, FLINT.top_k, fm.FLINT_SPLIT)
    s.ws = r.ws
    for i, (b, runner) in enumerate([(1, r), (8, r), (1, s), (1, r), (3, s), (3, r), (1, r), (8, s), (2, r)]):
        run_decode_case(DecodeCase(FLINT, seed=800 + i, batch=b), src=src, layer=layer, runner=runner)
    assert fm.decode_error_word(r) == 0


def test_fused_error_word_stays_clear():
    src = gen.moe_layer_source(FLINT, 602)
    layer = pack(src)
    r = fm.DecodeRunner(layer, FLINT.top_k, 0)
    for b in (1, 8):
        x = gen.activations(9, b, FLINT.hidden).cuda()
        for _ in range(20):
            r(x)
    torch.cuda.synchronize()
    assert fm.decode_error_word(r) == 0


def test_bounded_wait_gives_up_and_sets_error_word():
    """A wait limit of one reload, stored in the workspace header by the host,
    makes the single-launch kernel's waits give up before most hand-off words
    arrive: the kernel still exits and reports it in the error word.  Once the
    workspace is zero-filled again, calls give the normal result."""
    src = gen.moe_layer_source(FLINT, 604)
    layer = pack(src)
    for stack, batch in ((False, 1), (True, 1), (False, 8)):
        r = fm.DecodeRunner(layer, FLINT.top_k, fm.FLINT_PRE_RMSNORM | fm.FLINT_RESIDUAL)
        gamma = gen.rmsnorm_gamma(13, FLINT.hidden, "cuda")
        step = fm.DecodeStep([layer, layer], [gamma, gamma], [], [], FLINT.top_k, stack=True)
        step.ws = r.ws
        x = gen.activations(12, batch, FLINT.hidden).cuda()

        def call():
            if stack:
                y = x.clone()
                step(y)
                return y
            return r(x, gamma=gamma)

        want = call().clone()
        torch.cuda.synchronize()
        assert fm.decode_error_word(r) == 0
        lim = r.ws[fm.WS_WAIT_LIMIT_OFFSET:fm.WS_WAIT_LIMIT_OFFSET + 4].view(torch.int32)
        lim.fill_(1)
        call()
        torch.cuda.synchronize()
        assert fm.decode_error_word(r) == 1, f"stack={stack} batch={batch}"
        r.ws.zero_()
        got = call()
        torch.cuda.synchronize()
        assert fm.decode_error_word(r) == 0
        assert torch.equal(got, want)
