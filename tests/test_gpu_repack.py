"""Repack / unpack / dequant on the GPU against the oracle's source decode
(bit-exact), through the C ABI."""
import numpy as np
import pytest
import torch

import gen
import w4a16_moe_decode_amd as fm
from oracle import formats

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layout", gen.SRC_LAYOUTS)
@pytest.mark.parametrize("scale_mode", ["pow2", "full", "bytes"])
@pytest.mark.parametrize("rows,cols,n", [(8, 64, 1), (37, 192, 3), (128, 2048, 2)])
def test_repack_roundtrip_and_dequant_bitexact(layout, scale_mode, rows, cols, n):
    src = gen.nvfp4_source(gen.seed_for(1, layout, scale_mode, rows), n, rows, cols, "cpu", layout,
                           scale_mode)
    d = src.cuda()
    codes, scales = fm.repack_matrices(d, layout)
    back = torch.empty_like(d)
    fm.flint_moe_unpack(codes, scales, n, rows, cols, fm.SRC_LAYOUT_CODES[layout], 1, back)
    ts = torch.tensor([0.015625, 0.0123, 3.0][:n] + [1.0] * max(0, n - 3), dtype=torch.float32).cuda()
    deq = torch.empty((n, rows, cols), dtype=torch.float32, device="cuda")
    fm.flint_nvfp4_dequant(codes, scales, n, rows, cols, ts, deq)
    torch.cuda.synchronize()
    assert torch.equal(back.cpu(), src), "unpack(repack(src)) != src"
    # the packed planes hold exactly the documented layout
    c = codes.cpu().numpy().reshape(n, rows, cols // 2)
    s = scales.cpu().numpy().reshape(n, rows, cols // 16)
    sc, cd = formats.split_superblocks(src.numpy(), layout)
    np.testing.assert_array_equal(s, sc.reshape(n, rows, cols // 16))
    np.testing.assert_array_equal(c, cd.reshape(n, rows, cols // 2))
    got = deq.cpu().numpy()
    for m in range(n):
        want = formats.decode_source_matrix(src[m].numpy(), layout, float(ts[m])).astype(np.float32)
        nan = np.isnan(want)
        np.testing.assert_array_equal(np.isnan(got[m]), nan)
        np.testing.assert_array_equal(got[m][~nan], want[~nan])


def test_repack_matrix_stride_interleaves_gate_and_up():
    E, I, H = 3, 64, 128
    g = gen.nvfp4_source(5, E, I, H)
    u = gen.nvfp4_source(6, E, I, H)
    cb, sb = fm.flint_nvfp4_packed_bytes(2 * E, I, H)
    codes = torch.zeros(cb, dtype=torch.uint8, device="cuda")
    scales = torch.zeros(sb, dtype=torch.uint8, device="cuda")
    fm.repack_matrices(g.cuda(), "interleaved", codes, scales, 2)
    fm.repack_matrices(u.cuda(), "interleaved", codes[I * H // 2:], scales[I * H // 16:], 2)
    deq = torch.empty((2 * E, I, H), dtype=torch.float32, device="cuda")
    fm.flint_nvfp4_dequant(codes, scales, 2 * E, I, H, None, deq)
    torch.cuda.synchronize()
    got = deq.cpu().numpy()
    for e in range(E):
        np.testing.assert_array_equal(got[2 * e], formats.decode_source_matrix(g[e].numpy()))
        np.testing.assert_array_equal(got[2 * e + 1], formats.decode_source_matrix(u[e].numpy()))
