"""Prefill MoE layer (flint_moe_prefill: router GEMM, top-k, stable
permutation by expert, grouped GEMMs on MFMA, combine) on the GPU against
the oracle's per-token definition.  Routing is checked for every token;
outputs for every token at small sizes and for a sample of tokens at the
8,192-token size."""
import numpy as np
import pytest
import torch

import gen
import w4a16_moe_decode_amd as fm
from _parity import check_routing, compare_outputs, oracle_experts, pack
from oracle import bf16 as obf
from oracle import moe

pytestmark = pytest.mark.gpu

TINY = gen.SHAPE_TINY
FLINT = gen.SHAPE_FLINT


def run_prefill(shape, src, layer, T, seed, flags=0, x_kind="iid", sample=None, wbf16=False):
    x = gen.activations(gen.seed_for(seed, "px", T), T, shape.hidden, "cpu", x_kind)
    gamma = gen.rmsnorm_gamma(gen.seed_for(seed, "pg"), shape.hidden)
    f = flags | (fm.FLINT_W_BF16 if wbf16 else 0)
    runner = fm.PrefillRunner(layer, shape.top_k, T, f)
    idx = torch.full((T, shape.top_k), -1, dtype=torch.int32, device="cuda")
    wts = torch.zeros((T, shape.top_k), dtype=torch.float32, device="cuda")
    out = runner(x.cuda(), topk_idx=idx, topk_w=wts, gamma=gamma.cuda())
    torch.cuda.synchronize()
    ex = oracle_experts(src)
    xo = gen.numpy_f64(x)
    renorm = bool(flags & fm.FLINT_RENORM)
    xin = moe.rmsnorm(xo, gen.numpy_f64(gamma)) if flags & fm.FLINT_PRE_RMSNORM else xo
    # routing of every token
    r = moe.route(xin, ex.router, shape.top_k, renorm)
    idx_np = idx.cpu().numpy()
    forced = check_routing(idx_np, wts.cpu().numpy(), r, renorm)
    if callable(sample):
        sample = sample(idx_np)
    toks = np.arange(T) if sample is None else np.asarray(sample)
    want, _ = moe.moe_layer(xin[toks], ex, shape.top_k, renorm, forced_idx=forced[toks])
    if flags & fm.FLINT_RESIDUAL:
        want = obf.round_bf16(xo[toks] + want)
    compare_outputs(gen.numpy_f64(out)[toks], want)
    return idx.cpu().numpy()


@pytest.mark.parametrize("T", [1, 7, 64, 130, 333])
@pytest.mark.parametrize("renorm", [False, True])
def test_tiny_prefill(T, renorm):
    src = gen.moe_layer_source(TINY, 31)
    run_prefill(TINY, src, pack(src), T, 32, fm.FLINT_RENORM if renorm else 0)


@pytest.mark.parametrize("shape,T", [
    (gen.MoeShape(hidden=576, n_experts=40, inter=192, shared_inter=320, top_k=5), 97),
    (gen.MoeShape(hidden=256, n_experts=16, inter=64, shared_inter=0, top_k=8), 150),
    (gen.MoeShape(hidden=64, n_experts=1, inter=64, shared_inter=64, top_k=1), 5),
])
def test_ragged_prefill(shape, T):
    src = gen.moe_layer_source(shape, 33)
    layer = pack(src)
    run_prefill(shape, src, layer, T, 34)
    layer.add_bf16()
    run_prefill(shape, src, layer, T, 35, wbf16=True)


def test_prefill_norm_residual_and_skew():
    src = gen.moe_layer_source(TINY, 36)
    idx = run_prefill(TINY, src, pack(src), 300, 37, fm.FLINT_PRE_RMSNORM | fm.FLINT_RESIDUAL,
                      x_kind="correlated")
    h = np.bincount(idx.reshape(-1), minlength=TINY.n_experts)
    assert h.sum() == 300 * TINY.top_k and h.max() > 2 * h.mean()   # skewed histogram


@pytest.fixture(scope="module")
def flint():
    src = gen.moe_layer_source(FLINT, 200, "cpu")
    return src, pack(src)


def test_flint_prefill_1024(flint):
    src, layer = flint
    run_prefill(FLINT, src, layer, 1024, 38, sample=np.arange(0, 1024, 7))


TILE_ROWS = 128          # rows of one grouped-GEMM M-tile


def tile_edge_tokens(idx: np.ndarray, with_shared: bool = True) -> np.ndarray:
    """The tokens in the first and the last row of every M-tile of the
    grouped GEMMs.  Expert e's rows are its (token, slot) pairs in token
    order (the stable permutation by expert, then token), cut into tiles of
    128 rows; the shared expert's rows are all tokens in order.  ``idx`` is
    the GPU's routing, already checked against the oracle token by token."""
    T = idx.shape[0]
    out = set()
    for e in np.unique(idx):
        toks = np.nonzero((idx == e).any(1))[0]
        for m0 in range(0, len(toks), TILE_ROWS):
            out.add(int(toks[m0]))
            out.add(int(toks[min(m0 + TILE_ROWS, len(toks)) - 1]))
    if with_shared:
        for m0 in range(0, T, TILE_ROWS):
            out.update((m0, min(m0 + TILE_ROWS, T) - 1))
    return np.array(sorted(out))


@pytest.mark.parametrize("x_kind", ["iid", "correlated"])
def test_flint_prefill_8192(flint, x_kind):
    """Every M-tile of every expert group (several per expert, up to ~25 for
    the hottest expert under skew) and of the shared group has its first and
    last row compared with the oracle."""
    src, layer = flint
    seen = {}

    def sample(idx):
        seen["toks"] = tile_edge_tokens(idx)
        return seen["toks"]

    idx = run_prefill(FLINT, src, layer, 8192, 39, fm.FLINT_RENORM, x_kind=x_kind, sample=sample)
    h = np.bincount(idx.reshape(-1), minlength=FLINT.n_experts)
    assert h.sum() == 8192 * FLINT.top_k
    n_tiles = sum((c + TILE_ROWS - 1) // TILE_ROWS for c in h) + 8192 // TILE_ROWS
    assert len(seen["toks"]) >= min(n_tiles, 8192) // 2
    if x_kind == "correlated":
        assert h.max() > 4 * TILE_ROWS          # several M-tiles for one expert


def test_prefill_matches_decode(flint):
    """Prefill of a few tokens equals decode of the same tokens (same
    definition; only fp32 summation order may differ)."""
    src, layer = flint
    x = gen.activations(40, 8, FLINT.hidden).cuda()
    d = fm.DecodeRunner(layer, FLINT.top_k, 0)(x)
    p = fm.PrefillRunner(layer, FLINT.top_k, 8, 0)(x)
    torch.cuda.synchronize()
    compare_outputs(gen.numpy_f64(p), gen.numpy_f64(d), "prefill vs decode")


def test_prefill_bit_reproducible(flint):
    src, layer = flint
    x = gen.activations(41, 700, FLINT.hidden).cuda()
    r = fm.PrefillRunner(layer, FLINT.top_k, 700, 0)
    a = r(x).clone()
    b = r(x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------- the prefill layout --

def prefill_layout_reference(codes: np.ndarray, scales: np.ndarray, rows: int, cols: int,
                             interleave: int):
    """flint_moe_prefill_layout's definition (include/flint_moe.h), written
    out block by block: 32 virtual rows x 128 columns per block; virtual row
    2 i + u of a pair set is row i of matrix u (interleave), else row v."""
    n_mats = codes.shape[0] // (rows * cols // 2)
    c = codes.reshape(n_mats, rows, cols // 2)
    s = scales.reshape(n_mats, rows, cols // 16)
    per = 1 + interleave
    n_sets, rv, nkb = n_mats // per, rows * per, cols // 128
    oc = np.zeros_like(codes).reshape(n_sets, rv // 32, nkb, 2048)
    os_ = np.zeros_like(scales).reshape(n_sets, rv // 32, nkb, 256)
    for m in range(n_sets):
        for v in range(rv):
            mat, row = (per * m + v % 2, v // 2) if interleave else (m, v)
            vb, n = divmod(v, 32)
            for kb in range(nkb):
                for h in range(2):
                    for p in range(2):
                        src = c[mat, row, 64 * kb + 32 * h + 16 * p: 64 * kb + 32 * h + 16 * p + 16]
                        oc[m, vb, kb, 1024 * p + 16 * (2 * n + h): 1024 * p + 16 * (2 * n + h) + 16] = src
                    os_[m, vb, kb, 4 * (2 * n + h): 4 * (2 * n + h) + 4] = s[mat, row, 8 * kb + 4 * h: 8 * kb + 4 * h + 4]
    return oc.reshape(-1), os_.reshape(-1)


@pytest.mark.parametrize("n_mats,rows,cols,interleave", [(3, 64, 256, 0), (4, 48, 384, 1), (2, 16, 128, 1)])
def test_prefill_layout_matches_definition(n_mats, rows, cols, interleave):
    g = torch.Generator().manual_seed(n_mats * 1000 + rows + cols + interleave)
    codes = torch.randint(0, 256, (n_mats * rows * cols // 2,), generator=g, dtype=torch.uint8)
    scales = torch.randint(0, 256, (n_mats * rows * cols // 16,), generator=g, dtype=torch.uint8)
    oc = torch.empty_like(codes, device="cuda")
    os_ = torch.empty_like(scales, device="cuda")
    fm.flint_moe_prefill_layout(codes.cuda(), scales.cuda(), n_mats, rows, cols, interleave, oc, os_)
    torch.cuda.synchronize()
    wc, ws_ = prefill_layout_reference(codes.numpy(), scales.numpy(), rows, cols, interleave)
    assert np.array_equal(oc.cpu().numpy(), wc)
    assert np.array_equal(os_.cpu().numpy(), ws_)


def _prefill_pair(layer, shape, T, seed, flags=0, x_kind="iid"):
    """The same call through flint_moe_prefill and flint_moe_prefill_tiled."""
    x = gen.activations(gen.seed_for(seed, "tx", T), T, shape.hidden, "cuda", x_kind)
    gamma = gen.rmsnorm_gamma(gen.seed_for(seed, "tg"), shape.hidden).cuda()
    res = []
    for tiled in (False, True):
        runner = fm.PrefillRunner(layer, shape.top_k, T, flags, tiled=tiled)
        idx = torch.full((T, shape.top_k), -1, dtype=torch.int32, device="cuda")
        wts = torch.zeros((T, shape.top_k), dtype=torch.float32, device="cuda")
        out = runner(x, topk_idx=idx, topk_w=wts, gamma=gamma)
        torch.cuda.synchronize()
        res.append((out.cpu(), idx.cpu(), wts.cpu()))
    return res


@pytest.mark.parametrize("T,flags,x_kind", [
    (1, 0, "iid"), (100, fm.FLINT_RENORM, "iid"), (2048, fm.FLINT_PRE_RMSNORM | fm.FLINT_RESIDUAL, "iid"),
    (8192, fm.FLINT_RENORM, "correlated")])
def test_flint_prefill_tiled_is_bit_identical(flint, T, flags, x_kind):
    """The prefill layout changes only where the grouped GEMMs read their
    weights from: outputs, indices and weights equal the packed-plane path's
    bit for bit (that path is checked against the oracle above)."""
    _, layer = flint
    (o0, i0, w0), (o1, i1, w1) = _prefill_pair(layer, FLINT, T, 40 + T, flags, x_kind)
    assert torch.equal(i0, i1) and torch.equal(w0, w1)
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))


def test_flint_prefill_tiled_against_oracle(flint):
    src, layer = flint
    T = 333
    x = gen.activations(gen.seed_for(41, "px", T), T, FLINT.hidden, "cpu", "iid")
    runner = fm.PrefillRunner(layer, FLINT.top_k, T, 0, tiled=True)
    idx = torch.full((T, FLINT.top_k), -1, dtype=torch.int32, device="cuda")
    wts = torch.zeros((T, FLINT.top_k), dtype=torch.float32, device="cuda")
    out = runner(x.cuda(), topk_idx=idx, topk_w=wts)
    torch.cuda.synchronize()
    ex = oracle_experts(src)
    xo = gen.numpy_f64(x)
    r = moe.route(xo, ex.router, FLINT.top_k, False)
    forced = check_routing(idx.cpu().numpy(), wts.cpu().numpy(), r, False)
    want, _ = moe.moe_layer(xo, ex, FLINT.top_k, False, forced_idx=forced)
    compare_outputs(gen.numpy_f64(out), want)


def test_prefill_planes_ignored_at_other_shapes():
    src = gen.moe_layer_source(TINY, 42)
    layer = pack(src)
    (o0, i0, w0), (o1, i1, w1) = _prefill_pair(layer, TINY, 130, 43, fm.FLINT_RENORM)
    assert torch.equal(i0, i1) and torch.equal(w0, w1)
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
