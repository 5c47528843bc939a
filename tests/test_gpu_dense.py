"""Dense GEMV (flint_dense_gemv) on the GPU against the oracle: the SwiGLU
gate/up pair (with and without the fused RMSNorm), the plain projection and
the residual projection, NVFP4 and BF16 weights, the 2048 -> 5632 -> 2048
dense MLP shape and ragged shapes."""
import numpy as np
import pytest
import torch

import gen
import w4a16_moe_decode_amd as fm
from _parity import compare_outputs
from oracle import bf16 as obf
from oracle import formats, moe

pytestmark = pytest.mark.gpu


def _pack_pair(g_src, u_src):
    """gate and up sources [1][R][C/64][36] -> planes [2][R][C] on the GPU."""
    _, R, nb, _ = g_src.shape
    C = nb * 64
    cb, sb = fm.flint_nvfp4_packed_bytes(2, R, C)
    codes = torch.empty(cb, dtype=torch.uint8, device="cuda")
    scales = torch.empty(sb, dtype=torch.uint8, device="cuda")
    fm.repack_matrices(g_src.cuda(), "interleaved", codes, scales)
    fm.repack_matrices(u_src.cuda(), "interleaved", codes[R * C // 2:], scales[R * C // 16:])
    return codes, scales


def _bf16_of(src, ts):
    return torch.tensor(formats.decode_source_matrix(src[0].numpy(), "interleaved", ts),
                        dtype=torch.float32).to(torch.bfloat16).cuda()


@pytest.mark.parametrize("rows,cols,batch", [(5632, 2048, 1), (5632, 2048, 8), (960, 2048, 3), (320, 4096, 1),
                                             (320, 4096, 2), (192, 320, 3), (64, 64, 2)])
@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("wbf16", [False, True])
def test_swiglu_pair(rows, cols, batch, norm, wbf16):
    g_src, u_src, _, ts = gen.dense_mlp_source(cols, rows, gen.seed_for(7, rows, cols, batch))
    ts = ts.reshape(-1)
    x = gen.activations(gen.seed_for(8, rows), batch, cols)
    gamma = gen.rmsnorm_gamma(9, cols)
    y = torch.empty((batch, rows), dtype=torch.bfloat16, device="cuda")
    flags = (fm.FLINT_PRE_RMSNORM if norm else 0) | (fm.FLINT_W_BF16 if wbf16 else 0)
    gs = ts[:2].clone().cuda()
    if wbf16:
        w = torch.stack([_bf16_of(g_src, float(ts[0])), _bf16_of(u_src, float(ts[1]))]).contiguous()
        fm.flint_dense_gemv(None, None, None, w, rows, cols, flags, x.cuda(), batch, y,
                            fm.FLINT_EPI_SWIGLU, gamma=gamma.cuda(), rms_eps=1e-6)
    else:
        codes, scales = _pack_pair(g_src, u_src)
        fm.flint_dense_gemv(codes, scales, gs, None, rows, cols, flags, x.cuda(), batch, y,
                            fm.FLINT_EPI_SWIGLU, gamma=gamma.cuda(), rms_eps=1e-6)
    torch.cuda.synchronize()
    xo = gen.numpy_f64(x)
    if norm:
        xo = moe.rmsnorm(xo, gen.numpy_f64(gamma), 1e-6)
    wg = formats.decode_source_matrix(g_src[0].numpy(), "interleaved", float(ts[0]))
    wu = formats.decode_source_matrix(u_src[0].numpy(), "interleaved", float(ts[1]))
    wd = np.zeros((1, rows))
    want = np.stack([moe.expert_ffn(xo[t], wg, wu, wd)[1][2] for t in range(batch)])
    compare_outputs(gen.numpy_f64(y), want, "h")


@pytest.mark.parametrize("rows,cols,batch", [(2048, 5632, 1), (2048, 5632, 8), (136, 192, 5)])
@pytest.mark.parametrize("epi", [fm.FLINT_EPI_NONE, fm.FLINT_EPI_RESIDUAL])
@pytest.mark.parametrize("wbf16", [False, True])
def test_projection(rows, cols, batch, epi, wbf16):
    ts = gen.tensor_scales(gen.seed_for(10, rows, cols), 1, "varied")
    d_src = gen.nvfp4_source(gen.seed_for(11, rows, cols), 1, rows, cols)
    t0 = float(ts.reshape(-1)[2])
    x = gen.activations(gen.seed_for(12, cols), batch, cols)
    aux = gen.activations(gen.seed_for(13, rows), batch, rows)
    y = torch.empty((batch, rows), dtype=torch.bfloat16, device="cuda")
    gs = torch.tensor([t0, 0, 0, 0], dtype=torch.float32).cuda()
    auxd = aux.cuda() if epi == fm.FLINT_EPI_RESIDUAL else None
    if wbf16:
        w = _bf16_of(d_src, t0)
        fm.flint_dense_gemv(None, None, None, w, rows, cols, fm.FLINT_W_BF16, x.cuda(), batch, y, epi,
                            aux=auxd)
        wd = gen.numpy_f64(w.cpu())          # the BF16 weights as given
    else:
        codes, scales = fm.repack_matrices(d_src.cuda())
        fm.flint_dense_gemv(codes, scales, gs, None, rows, cols, 0, x.cuda(), batch, y, epi, aux=auxd)
        wd = formats.decode_source_matrix(d_src[0].numpy(), "interleaved", t0)
    torch.cuda.synchronize()
    want = obf.round_bf16(gen.numpy_f64(x) @ wd.T)
    if epi == fm.FLINT_EPI_RESIDUAL:
        want = obf.round_bf16(gen.numpy_f64(aux) + want)
    compare_outputs(gen.numpy_f64(y), want, "y")


def test_residual_in_place():
    rows, cols, batch = 256, 512, 4
    d_src = gen.nvfp4_source(21, 1, rows, cols)
    codes, scales = fm.repack_matrices(d_src.cuda())
    gs = torch.tensor([1 / 64, 0, 0, 0], dtype=torch.float32).cuda()
    x = gen.activations(22, batch, cols).cuda()
    aux = gen.activations(23, batch, rows)
    y = aux.clone().cuda()
    fm.flint_dense_gemv(codes, scales, gs, None, rows, cols, 0, x, batch, y, fm.FLINT_EPI_RESIDUAL, aux=y)
    torch.cuda.synchronize()
    wd = formats.decode_source_matrix(d_src[0].numpy(), "interleaved", 1 / 64)
    want = obf.round_bf16(gen.numpy_f64(aux) + obf.round_bf16(gen.numpy_f64(x.cpu()) @ wd.T))
    compare_outputs(gen.numpy_f64(y), want, "y")


@pytest.mark.parametrize("rows,cols,batch", [(1000, 2048, 1), (1000, 2048, 5), (333, 4096, 8), (64, 4096, 1)])
@pytest.mark.parametrize("epi", [fm.FLINT_EPI_NONE, fm.FLINT_EPI_RESIDUAL])
def test_tall_projection_shapes(rows, cols, batch, epi):
    """The tall-matrix NVFP4 projection (2048 or 4096 columns): ragged row
    counts, every batch size class, both epilogues, non-power-of-two scale."""
    ts = gen.tensor_scales(gen.seed_for(30, rows, cols), 1, "varied")
    d_src = gen.nvfp4_source(gen.seed_for(31, rows, cols), 1, rows, cols, scale_mode="full")
    t0 = float(ts.reshape(-1)[2])
    x = gen.activations(gen.seed_for(32, cols, batch), batch, cols)
    aux = gen.activations(gen.seed_for(33, rows, batch), batch, rows)
    y = torch.empty((batch, rows), dtype=torch.bfloat16, device="cuda")
    gs = torch.tensor([t0, 0, 0, 0], dtype=torch.float32).cuda()
    codes, scales = fm.repack_matrices(d_src.cuda())
    auxd = aux.cuda() if epi == fm.FLINT_EPI_RESIDUAL else None
    fm.flint_dense_gemv(codes, scales, gs, None, rows, cols, 0, x.cuda(), batch, y, epi, aux=auxd)
    torch.cuda.synchronize()
    wd = formats.decode_source_matrix(d_src[0].numpy(), "interleaved", t0)
    want = obf.round_bf16(gen.numpy_f64(x) @ wd.T)
    if epi == fm.FLINT_EPI_RESIDUAL:
        want = obf.round_bf16(gen.numpy_f64(aux) + want)
    compare_outputs(gen.numpy_f64(y), want, "y")


LM_HEAD_ROWS = 150144      # vocabulary rows of an NVFP4 LM head over hidden 2048


@pytest.mark.parametrize("batch", [1, 8])
def test_lm_head_projection_sampled(batch):
    """The LM-head shape (2048 -> 150,144, 173 MB of NVFP4 weights) in the
    launch configuration the benchmark times, checked against the oracle on
    a sample of rows (every 151st row plus the ragged tail), which the
    oracle decodes from the source bytes."""
    rows, cols = LM_HEAD_ROWS, 2048
    d_src = gen.nvfp4_source(gen.seed_for(40, batch), 1, rows, cols)
    x = gen.activations(gen.seed_for(41, batch), batch, cols)
    y = torch.empty((batch, rows), dtype=torch.bfloat16, device="cuda")
    gs = torch.tensor([1 / 64, 0, 0, 0], dtype=torch.float32).cuda()
    codes, scales = fm.repack_matrices(d_src.cuda())
    fm.flint_dense_gemv(codes, scales, gs, None, rows, cols, 0, x.cuda(), batch, y, fm.FLINT_EPI_NONE)
    torch.cuda.synchronize()
    sample = np.unique(np.concatenate([np.arange(0, rows, 151), np.arange(rows - 70, rows)]))
    wd = formats.decode_source_matrix(d_src[0, torch.from_numpy(sample)].numpy(), "interleaved", 1 / 64)
    want = obf.round_bf16(gen.numpy_f64(x) @ wd.T)
    compare_outputs(gen.numpy_f64(y.cpu())[:, sample], want, "y")
