"""Shared helpers of the GPU parity tests: build a layer from the seeded
generators, run it through the C ABI, run the oracle on the same inputs and
compare with the stated bars.

Bars (fixed before any kernel was written):
  * repack: bit-exact; dequant: bit-exact in float32
  * expert indices: exact, except for tokens whose oracle gap between the
    k-th and (k+1)-th sigmoid score is below 1e-5 -- there the GPU's choice
    must be a valid top-k (checked by re-running the oracle on it)
  * outputs, per token: max|gpu - oracle| <= 1e-2 * max|oracle| and
    cosine(gpu, oracle) >= 0.9999
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import gen
import w4a16_moe_decode_amd as fm
from oracle import formats, moe

GAP_EXEMPT = 1e-5
REL_TOL = 1e-2
COS_MIN = 0.9999


def oracle_experts(src: gen.MoeLayerSource) -> moe.ExpertSet:
    u8 = gen.numpy_u8
    sh = src.sh_gate is not None
    return moe.nvfp4_expert_set(
        gen.numpy_f64(src.router), u8(src.gate), u8(src.up), u8(src.down), src.gscale.numpy(),
        u8(src.sh_gate) if sh else None, u8(src.sh_up) if sh else None,
        u8(src.sh_down) if sh else None, src.sh_gscale.numpy(), src.layout)


def oracle_experts_lazy(src: gen.MoeLayerSource) -> moe.ExpertSet:
    """Oracle expert set over a source layer that may live on the GPU: an
    expert's bytes are copied to the host only when the oracle asks for it."""
    gs = src.gscale.cpu().numpy().astype(np.float64)
    sg = src.sh_gscale.cpu().numpy().astype(np.float64).reshape(3)
    dec = lambda t, g: formats.decode_source_matrix(t.cpu().numpy(), src.layout, g)

    def load(e):
        if e is None:
            if src.sh_gate is None:
                return None
            return dec(src.sh_gate[0], sg[0]), dec(src.sh_up[0], sg[1]), dec(src.sh_down[0], sg[2])
        return dec(src.gate[e], gs[e, 0]), dec(src.up[e], gs[e, 1]), dec(src.down[e], gs[e, 2])

    return moe.ExpertSet(router=gen.numpy_f64(src.router), n_experts=src.router.shape[0], _loader=load)


def pack(src: gen.MoeLayerSource, device="cuda") -> fm.PackedMoeLayer:
    return fm.pack_moe_layer(src.router, src.gate, src.up, src.down, src.gscale, src.sh_gate,
                             src.sh_up, src.sh_down, src.sh_gscale, src.layout, device)


def _nan_positions(got: np.ndarray, want: np.ndarray, what: str):
    """Non-finite values are allowed only where the oracle has NaN (a NaN
    scale byte propagates through the expert that uses it), and there the
    GPU must have NaN too.  Returns the mask of positions to compare."""
    want_nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), want_nan), \
        f"{what}: NaN at {np.argwhere(np.isnan(got) != want_nan)[:8].tolist()} differs from the oracle"
    assert np.all(np.isfinite(got[~want_nan])), f"{what}: non-finite GPU values"
    return ~want_nan


def compare_outputs(got: np.ndarray, want: np.ndarray, what: str = "out"):
    got = np.atleast_2d(got)
    want = np.atleast_2d(want)
    assert got.shape == want.shape, (got.shape, want.shape)
    live = _nan_positions(got, want, what)
    for t in range(want.shape[0]):
        g, w = got[t][live[t]], want[t][live[t]]
        if g.size == 0:
            continue
        scale = np.max(np.abs(w))
        err = np.max(np.abs(g - w))
        if scale == 0.0:
            assert err == 0.0, f"{what}[{t}]: oracle is all zero, GPU max|d|={err:.4g}"
            continue
        assert err <= REL_TOL * scale, f"{what}[{t}]: max|d|={err:.4g} > {REL_TOL}*{scale:.4g}"
        cos = float(g @ w / (np.linalg.norm(g) * np.linalg.norm(w) + 1e-300))
        assert cos >= COS_MIN, f"{what}[{t}]: cosine {cos:.6f}"


def bf16_ulp(v):
    """Spacing of bfloat16 values at |v| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(int) - 7)


def compare_residual(got_out: np.ndarray, want_out: np.ndarray, x_in: np.ndarray, what: str):
    """A sublayer that updates the residual, x_out = BF16(x_in + y): the
    update y is held to the output bar, plus one BF16 ulp of x_out, since a
    last-bit difference in y can move the rounding of the sum by one ulp."""
    got_out, want_out, x_in = (np.atleast_2d(a) for a in (got_out, want_out, x_in))
    live = _nan_positions(got_out, want_out, what)
    for t in range(want_out.shape[0]):
        m = live[t]
        dg, dw = got_out[t][m] - x_in[t][m], want_out[t][m] - x_in[t][m]
        scale = np.max(np.abs(dw)) if dw.size else 0.0
        err = np.abs(got_out[t][m] - want_out[t][m])
        allow = REL_TOL * scale + bf16_ulp(want_out[t][m])
        assert np.all(err <= allow), f"{what}[{t}]: max excess {np.max(err - allow):.4g}"
        if scale == 0.0:
            continue
        cos = float(dg @ dw / (np.linalg.norm(dg) * np.linalg.norm(dw) + 1e-300))
        assert cos >= COS_MIN, f"{what}[{t}]: cosine {cos:.6f}"


def check_routing(idx_gpu: np.ndarray, w_gpu: np.ndarray, r: moe.Routing, renorm: bool):
    """Indices exact unless the oracle's gap is under GAP_EXEMPT; weights
    within fp32 accuracy.  Returns the per-token index sets to feed back to
    the oracle (its own, or the GPU's for exempt tokens)."""
    forced = r.idx.copy()
    for t in range(r.idx.shape[0]):
        if r.gap[t] >= GAP_EXEMPT:
            assert list(idx_gpu[t]) == list(r.idx[t]), f"token {t}: {idx_gpu[t]} vs {r.idx[t]}"
        else:
            # a valid top-k under the near-tie: the GPU's experts hold the k
            # largest scores up to the exemption gap
            s = np.where(np.isnan(r.scores[t]), -np.inf, r.scores[t])
            kth = np.sort(s)[::-1][r.idx.shape[1] - 1]
            assert len(set(idx_gpu[t])) == r.idx.shape[1]
            assert np.all(s[idx_gpu[t]] >= kth - GAP_EXEMPT)
            forced[t] = idx_gpu[t]
    sel = np.take_along_axis(r.scores, forced, 1)
    want_w = sel / sel.sum(1, keepdims=True) if renorm else sel
    np.testing.assert_allclose(w_gpu, want_w, rtol=2e-5, atol=1e-7)
    return forced


@dataclasses.dataclass
class DecodeCase:
    shape: gen.MoeShape
    seed: int = 0
    batch: int = 1
    flags: int = 0
    layout: str = "interleaved"
    scale_mode: str = "pow2"
    gscale_mode: str = "pow2"
    x_kind: str = "iid"
    zero_x: bool = False
    wbf16: bool = False


def run_decode_case(c: DecodeCase, src=None, layer=None, runner=None):
    """Run one decode case on the GPU and check it against the oracle."""
    sh = c.shape
    if src is None:
        src = gen.moe_layer_source(sh, c.seed, "cpu", c.layout, c.scale_mode, c.gscale_mode)
    if layer is None:
        layer = pack(src)
        if c.wbf16:
            layer.add_bf16()
    flags = c.flags | (fm.FLINT_W_BF16 if c.wbf16 else 0)
    if runner is None:
        runner = fm.DecodeRunner(layer, sh.top_k, flags)
    x = gen.activations(gen.seed_for(c.seed, "x", c.batch), c.batch, sh.hidden, "cpu", c.x_kind)
    if c.zero_x:
        x.zero_()
    gamma = gen.rmsnorm_gamma(gen.seed_for(c.seed, "gamma"), sh.hidden)
    dev = torch.device("cuda")
    xd = x.to(dev)
    gd = gamma.to(dev)
    idx = torch.full((c.batch, sh.top_k), -1, dtype=torch.int32, device=dev)
    wts = torch.zeros((c.batch, sh.top_k), dtype=torch.float32, device=dev)
    out = runner(xd, topk_idx=idx, topk_w=wts, gamma=gd)
    torch.cuda.synchronize()

    ex = oracle_experts(src)
    xo = gen.numpy_f64(x)
    renorm = bool(c.flags & fm.FLINT_RENORM)
    xin = moe.rmsnorm(xo, gen.numpy_f64(gamma)) if c.flags & fm.FLINT_PRE_RMSNORM else xo
    _, r = moe.moe_layer(xin, ex, sh.top_k, renorm)
    forced = check_routing(idx.cpu().numpy(), wts.cpu().numpy(), r, renorm)
    want, _ = moe.moe_layer(xin, ex, sh.top_k, renorm, forced_idx=forced)
    if c.flags & fm.FLINT_RESIDUAL:
        from oracle.bf16 import round_bf16
        want = round_bf16(xo + want)
    got = gen.numpy_f64(out)
    compare_outputs(got, want)
    return got, want, r
