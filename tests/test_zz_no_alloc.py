"""flint_moe_decode_noalloc -- the decode layer on the library's static
device scratch instead of a caller's workspace -- against flint_moe_decode
on the same inputs: two calls in a row, the second with a smaller input,
for the one-launch batch-1 and batch kernels and the three-kernel path."""
import numpy as np
import pytest
import torch

import gen
import w4a16_moe_decode_amd as fm
from _parity import compare_outputs, compare_residual, pack

pytestmark = pytest.mark.gpu

FLINT = gen.SHAPE_FLINT


def _pair(layer, shape, flags, batch, seed, gamma):
    """(no-alloc result, workspace result) of one call: outputs and top-k."""
    K = shape.top_k
    x = gen.activations(gen.seed_for(seed, "noalloc", batch), batch, shape.hidden, "cuda")
    s = layer.shape(K, flags)
    w = layer.weights()
    res = []
    for noalloc in (True, False):
        out = torch.empty_like(x)
        idx = torch.full((batch, K), -1, dtype=torch.int32, device="cuda")
        wt = torch.zeros((batch, K), dtype=torch.float32, device="cuda")
        if noalloc:
            fm.flint_moe_decode_noalloc(s, w, x, batch, out, idx, wt, gamma)
        else:
            fm.DecodeRunner(layer, K, flags)(x, out=out, topk_idx=idx, topk_w=wt, gamma=gamma)
        res.append((out, idx, wt))
    torch.cuda.synchronize()
    return x, res


@pytest.mark.parametrize("flags", [0, fm.FLINT_RENORM | fm.FLINT_PRE_RMSNORM | fm.FLINT_RESIDUAL, fm.FLINT_SPLIT])
def test_noalloc_matches_workspace_entry_point(flags):
    src = gen.moe_layer_source(FLINT, 950, "cuda")
    layer = pack(src)
    gamma = gen.rmsnorm_gamma(951, FLINT.hidden, "cuda")
    # batch 8, then batch 1, then 3: each call's input is smaller than the
    # first's and the scratch still holds the previous call's state
    for batch in (8, 1, 3):
        path = (fm.FLINT_PATH_SPLIT if flags & fm.FLINT_SPLIT else
                fm.FLINT_PATH_SINGLE_ONE if batch == 1 else fm.FLINT_PATH_SINGLE_BATCH)
        assert fm.flint_moe_decode_path(layer.shape(FLINT.top_k, flags), batch) == path
        x, ((o1, i1, w1), (o2, i2, w2)) = _pair(layer, FLINT, flags, batch, 952 + flags, gamma)
        assert torch.equal(i1, i2) and torch.equal(w1, w2), f"routing, batch {batch}"
        got, want = gen.numpy_f64(o1), gen.numpy_f64(o2)
        if flags & fm.FLINT_RESIDUAL:
            compare_residual(got, want, gen.numpy_f64(x), f"noalloc batch {batch}")
        else:
            compare_outputs(got, want, f"noalloc batch {batch}")
        assert torch.equal(o1, o2), f"batch {batch}: same kernels, same bits"


def test_noalloc_small_shape_then_rejects_oversized():
    shape = gen.SHAPE_TINY
    src = gen.moe_layer_source(shape, 953, "cpu")
    layer = pack(src)
    for batch in (4, 1):
        _, ((o1, i1, _), (o2, i2, _)) = _pair(layer, shape, 0, batch, 954, None)
        assert torch.equal(o1, o2) and torch.equal(i1, i2)
    # a layer whose decode workspace exceeds the scratch is refused before
    # anything is enqueued
    big = fm.FlintMoeShape(4096, 256, 8192, 8192, 8, 0, 1e-6)
    with pytest.raises(fm.FlintError) as e:
        fm.flint_moe_decode_noalloc(big, layer.weights(), torch.zeros((1, 4096), dtype=torch.bfloat16,
                                                                      device="cuda"), 1,
                                    torch.zeros((1, 4096), dtype=torch.bfloat16, device="cuda"), None, None, None)
    assert e.value.status == fm.FLINT_ERR_WORKSPACE
