"""The fused per-head Q/K RMSNorm + RoPE + KV-cache write on the GPU
(flint_qk_norm_rope_kv) against the oracle (oracle/attn.py), at the Flint
attention shape (GQA 32 query / 4 KV heads of dimension 128): decode batches,
a ragged count, an 8,192-token prefill, RoPE and NoPE layers, padding slots,
and positions or slots out of range."""
import numpy as np
import pytest
import torch

import gen
import w4a16_moe_decode_amd as fm
from oracle import attn

pytestmark = pytest.mark.gpu

SH = gen.ATTN_FLINT
D = SH.head_dim
N_POS = 600            # table rows (the 513-token window and some margin)


def _case(seed, T, rope, n_slots, pad_every=0, bad=None):
    dev = torch.device("cuda")
    rng = np.random.default_rng(seed)
    qkv = gen.attn_rows(gen.seed_for(seed, "qkv"), T, SH, dev)
    gq = gen.rmsnorm_gamma(gen.seed_for(seed, "gq"), D, dev)
    gk = gen.rmsnorm_gamma(gen.seed_for(seed, "gk"), D, dev)
    table = gen.rope_table(N_POS, D, device=dev)
    pos = rng.integers(0, N_POS, size=T).astype(np.int32)
    slots = rng.permutation(n_slots)[:T].astype(np.int32)
    if pad_every:
        slots[::pad_every] = -1
    if bad == "pos":
        pos[T // 2] = N_POS
    elif bad == "neg_pos":
        pos[T // 2] = -3
    elif bad == "slot":
        slots[T // 2] = n_slots
    sentinel = 0x3F80    # BF16 1.0
    kc = torch.full((n_slots, SH.n_kv_heads, D), 1.0, dtype=torch.bfloat16, device=dev)
    vc = torch.full_like(kc, 1.0)
    q = torch.full((T, SH.n_q_heads, D), 1.0, dtype=torch.bfloat16, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    shape = fm.FlintAttnShape(SH.n_q_heads, SH.n_kv_heads, D, fm.FLINT_ATTN_ROPE if rope else 0, 1e-6)
    fm.flint_qk_norm_rope_kv(shape, qkv, T, torch.from_numpy(pos).to(dev), table, N_POS,
                             torch.from_numpy(slots).to(dev), kc, vc, n_slots, gq, gk, q, err)
    torch.cuda.synchronize()
    # oracle on the same inputs; a token with an index out of range is left out
    ok = np.ones(T, dtype=bool)
    if bad in ("pos", "neg_pos") and rope:
        ok[T // 2] = False
    if bad == "slot":
        ok[T // 2] = False
    kc_w = np.ones((n_slots, SH.n_kv_heads, D))
    vc_w = np.ones_like(kc_w)
    sl = np.where(ok, slots, -1)
    q_w = attn.qk_norm_rope_kv(gen.numpy_f64(qkv)[ok], SH.n_q_heads, SH.n_kv_heads, D, pos[ok], sl[ok],
                               gen.numpy_f64(gq), gen.numpy_f64(gk), gen.numpy_f64(table), kc_w, vc_w,
                               1e-6, rope)
    got_q = gen.numpy_f64(q)
    np.testing.assert_array_equal(got_q[ok], q_w)
    if not ok.all():
        assert np.all(got_q[~ok] == 1.0), "a rejected token's q rows were written"
    np.testing.assert_array_equal(gen.numpy_f64(kc), kc_w)
    np.testing.assert_array_equal(gen.numpy_f64(vc), vc_w)
    assert int(err.item()) == (0 if ok.all() else 1)
    del sentinel


@pytest.mark.parametrize("T", [1, 8, 61])
@pytest.mark.parametrize("rope", [True, False])
def test_decode_and_ragged(T, rope):
    _case(10 + T, T, rope, n_slots=128, pad_every=5 if T > 4 else 0)


def test_prefill_8192_tokens():
    _case(11, 8192, True, n_slots=8192, pad_every=97)


@pytest.mark.parametrize("bad", ["pos", "neg_pos", "slot"])
def test_out_of_range_index_sets_error_and_skips_token(bad):
    _case(12, 16, True, n_slots=64, bad=bad)


def test_nope_ignores_positions():
    """Without FLINT_ATTN_ROPE the positions are not read: an out-of-range
    position is no error there."""
    _case(13, 16, False, n_slots=64, bad="pos")
