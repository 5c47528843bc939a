"""A stack of MoE sublayers in one launch (flint_moe_decode_stack) against
one flint_moe_decode call per sublayer: the same arithmetic, so every
layer's residual and selection must agree bit for bit.  The oracle check of
the 47-layer step (test_gpu_step.py) runs through the stack at batch 1."""
import pytest
import torch

import gen
import w4a16_moe_decode_amd as fm
from _parity import check_routing, compare_residual, oracle_experts_lazy
from oracle import moe

pytestmark = pytest.mark.gpu

SH = gen.SHAPE_FLINT


def _layers(n, seed, shape=SH):
    dev = torch.device("cuda")
    srcs, layers, gammas = [], [], []
    for l in range(n):
        src = gen.moe_layer_source(shape, gen.seed_for(seed, "stack", l), dev)
        layers.append(fm.pack_moe_layer(src.router, src.gate, src.up, src.down, src.gscale, src.sh_gate,
                                        src.sh_up, src.sh_down, src.sh_gscale, src.layout, dev))
        srcs.append(src)
        gammas.append(gen.rmsnorm_gamma(gen.seed_for(seed, "stack-g", l), shape.hidden, dev))
    return srcs, layers, gammas


def _run_both(layers, gammas, x0, flags, shape=SH):
    a = fm.DecodeStep(layers, gammas, [], [], shape.top_k, flags=flags, stack=True)
    b = fm.DecodeStep(layers, gammas, [], [], shape.top_k, flags=flags, stack=False)
    assert a.stack_shape is not None and b.stack_shape is None
    ra, rb = [], []
    xa, xb = x0.clone(), x0.clone()
    a(xa, record=ra)
    b(xb, record=rb)
    torch.cuda.synchronize()
    return a, b, xa, xb, ra, rb


@pytest.mark.parametrize("flags", [0, fm.FLINT_RENORM])
def test_stack_equals_per_layer_calls(flags):
    _, layers, gammas = _layers(5, 31 + flags)
    x0 = gen.activations(gen.seed_for(7, "stack-x", flags), 1, SH.hidden, "cuda")
    a, b, xa, xb, ra, rb = _run_both(layers, gammas, x0, flags)
    assert len(ra) == len(rb) == 5
    for l in range(5):
        assert torch.equal(ra[l], rb[l]), f"residual entering layer {l}"
        ia, wa = a.routing(l, 1)
        ib, wb = b.routing(l, 1)
        assert torch.equal(ia, ib) and torch.equal(wa, wb), f"routing of layer {l}"
    assert torch.equal(xa, xb)
    assert fm.decode_error_word(a) == 0


def test_stack_other_shapes_against_oracle():
    """Hidden 4096 (two chunks per lane) and a stack of one layer, checked
    teacher-forced against the oracle."""
    shape = gen.MoeShape(hidden=4096, n_experts=64, inter=256, shared_inter=512, top_k=6)
    for n in (1, 3):
        srcs, layers, gammas = _layers(n, 40 + n, shape)
        step = fm.DecodeStep(layers, gammas, [], [], shape.top_k, stack=True)
        assert step.stack_shape is not None
        x = gen.activations(gen.seed_for(9, "stack-x4096", n), 1, shape.hidden, "cuda")
        rec = []
        step(x, record=rec)
        rec.append(x.clone())
        torch.cuda.synchronize()
        for l in range(n):
            xin = gen.numpy_f64(rec[l])
            ex = oracle_experts_lazy(srcs[l])
            g = gen.numpy_f64(gammas[l])
            _, r = moe.moe_sublayer(xin, g, ex, shape.top_k, False)
            idx, wts = (t.cpu().numpy() for t in step.routing(l, 1))
            forced = check_routing(idx, wts, r, False)
            want, _ = moe.moe_sublayer(xin, g, ex, shape.top_k, False, forced_idx=forced)
            compare_residual(gen.numpy_f64(rec[l + 1]), want, xin, f"layer {l} of {n}")


def test_stack_graph_replay_and_shared_workspace():
    """The stack replays in a HIP graph with the same result every time, and
    single-layer calls on the same workspace keep working in between."""
    _, layers, gammas = _layers(4, 50)
    step = fm.DecodeStep(layers, gammas, [], [], SH.top_k)
    single = fm.DecodeRunner(layers[0], SH.top_k, fm.FLINT_PRE_RMSNORM | fm.FLINT_RESIDUAL)
    single.ws = step.ws
    x0 = gen.activations(11, 1, SH.hidden, "cuda")
    eager = x0.clone()
    step(eager)
    xg = x0.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(xg)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(xg)
    ref_single = None
    for i in range(4):
        xg.copy_(x0)
        g.replay()
        y = single(x0, gamma=gammas[0])
        torch.cuda.synchronize()
        assert torch.equal(xg, eager), f"replay {i}"
        if ref_single is None:
            ref_single = y.clone()
        assert torch.equal(y, ref_single)
    assert fm.decode_error_word(step) == 0
