"""The multi-layer decode step (47 MoE sublayers + 2 dense SwiGLU
sublayers, pre-norm RMSNorm with eps 1e-6, residual updated in place) on
the GPU, checked teacher-forced per sublayer: the oracle takes the GPU's
residual entering each sublayer and must reproduce the GPU's residual
leaving it.  BF16 is ill-conditioned over many layers (routing flips
compound), so the free-running end-to-end output is not compared."""
import numpy as np
import pytest
import torch

import gen
import w4a16_moe_decode_amd as fm
from _parity import check_routing, compare_residual, oracle_experts_lazy
from oracle import formats, moe

pytestmark = pytest.mark.gpu

SH = gen.SHAPE_FLINT


def _build(n_moe, n_dense, seed, wbf16=False):
    dev = torch.device("cuda")
    srcs, layers, gmo = [], [], []
    for l in range(n_moe):
        src = gen.moe_layer_source(SH, gen.seed_for(seed, "moe", l), dev)
        L = fm.pack_moe_layer(src.router, src.gate, src.up, src.down, src.gscale, src.sh_gate,
                              src.sh_up, src.sh_down, src.sh_gscale, src.layout, dev)
        if wbf16:
            L.add_bf16()
        srcs.append(src)
        layers.append(L)
        gmo.append(gen.rmsnorm_gamma(gen.seed_for(seed, "gm", l), SH.hidden, dev))
    dsrc, dl, gde = [], [], []
    for l in range(n_dense):
        g, u, d, ts = gen.dense_mlp_source(SH.hidden, gen.DENSE_INTER, gen.seed_for(seed, "dense", l), dev)
        D = fm.pack_dense_mlp(g, u, d, ts, device=dev)
        if wbf16:
            D.add_bf16()
        dsrc.append((g, u, d, ts))
        dl.append(D)
        gde.append(gen.rmsnorm_gamma(gen.seed_for(seed, "gd", l), SH.hidden, dev))
    return srcs, layers, gmo, dsrc, dl, gde


def _check_step(n_moe, n_dense, batch, seed, wbf16=False, flags=0, stack=None):
    srcs, layers, gmo, dsrc, dl, gde = _build(n_moe, n_dense, seed, wbf16)
    step = fm.DecodeStep(layers, gmo, dl, gde, SH.top_k, flags=flags, wbf16=wbf16, stack=stack)
    x = gen.activations(gen.seed_for(seed, "x"), batch, SH.hidden, "cuda")
    rec = []
    step(x, record=rec)
    rec.append(x.clone())
    torch.cuda.synchronize()
    renorm = bool(flags & fm.FLINT_RENORM)
    for l in range(n_moe):
        xin = gen.numpy_f64(rec[l])
        ex = oracle_experts_lazy(srcs[l])
        g = gen.numpy_f64(gmo[l])
        _, r = moe.moe_sublayer(xin, g, ex, SH.top_k, renorm)
        idx_t, w_t = step.routing(l, batch)
        idx, wts = idx_t.cpu().numpy(), w_t.cpu().numpy()
        forced = check_routing(idx, wts, r, renorm)
        want, _ = moe.moe_sublayer(xin, g, ex, SH.top_k, renorm, forced_idx=forced)
        compare_residual(gen.numpy_f64(rec[l + 1]), want, xin, f"moe layer {l}")
    for j in range(n_dense):
        xin = gen.numpy_f64(rec[n_moe + j])
        g_src, u_src, d_src, ts = dsrc[j]
        t = ts.reshape(-1).cpu().numpy().astype(np.float64)
        dec = lambda s, v: formats.decode_source_matrix(s[0].cpu().numpy(), "interleaved", v)
        want = moe.dense_sublayer(xin, gen.numpy_f64(gde[j]), dec(g_src, t[0]), dec(u_src, t[1]),
                                  dec(d_src, t[2]))
        compare_residual(gen.numpy_f64(rec[n_moe + j + 1]), want, xin, f"dense layer {j}")


def test_full_decode_step_batch1():
    _check_step(47, 2, 1, seed=1)


def test_decode_step_batch1_one_call_per_layer():
    """The batch-1 step without the layer stack (one decode call per layer)."""
    _check_step(4, 1, 1, seed=6, stack=False)


def test_decode_step_batch8_renorm():
    _check_step(6, 2, 8, seed=2, flags=fm.FLINT_RENORM)


def test_decode_step_bf16_weights():
    _check_step(3, 2, 3, seed=3, wbf16=True)


def test_decode_step_bf16_weights_batch1():
    """W16A16 at batch 1: each MoE sublayer one launch of the BF16 form."""
    _check_step(3, 2, 1, seed=5, wbf16=True)


def test_step_graph_replay_matches_eager():
    srcs, layers, gmo, dsrc, dl, gde = _build(4, 2, seed=4)
    step = fm.DecodeStep(layers, gmo, dl, gde, SH.top_k)
    x0 = gen.activations(5, 2, SH.hidden, "cuda")
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
    for _ in range(3):
        xg.copy_(x0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xg, eager)
