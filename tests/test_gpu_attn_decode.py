"""Decode attention with learned sinks (flint_decode_attention) against the
oracle ("Day-0 Support for Flint on vLLM", "Model architecture": GQA 32/4,
head dimension 128, a 513-token window on most layers and the whole
context on the rest, learned sinks; "Optimizations": a decode attention
kernel with sinks and sliding windows).

Tolerance, from the kernel's arithmetic: the softmax weights enter the V
product rounded to BF16 (relative error <= 2^-9 each, so the mixture moves
by at most 2^-9 sum_p w_p |v_p|) and the output is rounded to BF16 once
(2^-9 relative); scores, exponentials and sums in float32 add far less.
Each element must satisfy |gpu - ref| <= 2^-8 (|ref| + sum_p w_p |v_p|),
twice that bound."""
import numpy as np
import pytest
import torch

import gen
import w4a16_moe_decode_amd as fm
from oracle import attn

pytestmark = pytest.mark.gpu

DEV = "cuda"
SCALE = 1.0 / np.sqrt(128.0)


def _run(case, n_q, n_kv, window, max_len=None, stream=None):
    B = case.q.shape[0]
    max_len = int(case.seq_len.max()) if max_len is None else max_len
    shape = fm.FlintAttnShape(n_q, n_kv, 128, 0, 0.0)
    wsb = fm.flint_decode_attention_workspace_bytes(shape, window, B, max_len)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
    out = torch.full((B, n_q, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    fm.flint_decode_attention(shape, window, case.ring, SCALE, case.q, B, case.k_cache, case.v_cache, case.n_rows,
                              case.seq_base, case.seq_len, max_len, case.sinks, out, ws if wsb else None, wsb,
                              err, stream)
    torch.cuda.synchronize()
    return out, int(err.item())


def _oracle(case, window):
    f64 = gen.numpy_f64
    return attn.decode_attention(f64(case.q), f64(case.k_cache), f64(case.v_cache), case.seq_base.cpu().numpy(),
                                 case.seq_len.cpu().numpy(), case.ring, window, f64(case.sinks), SCALE,
                                 with_abs=True)


def _check(out, ref, mix, rows=None):
    got = gen.numpy_f64(out)
    if rows is not None:
        got, ref, mix = got[rows], ref[rows], mix[rows]
    bound = 2.0 ** -8 * (np.abs(ref) + mix)
    bad = np.abs(got - ref) > bound
    assert np.isfinite(got).all()
    assert not bad.any(), (f"{bad.sum()} of {bad.size} outside the bound; worst excess "
                           f"{np.max(np.abs(got - ref) - bound):.3g}")


def _case(seed, n_q, n_kv, lens, ring):
    print(f"[attn-decode] seed {seed} heads {n_q}/{n_kv} lens {list(lens)[:8]} ring {ring}", flush=True)
    return gen.decode_attn_case(seed, n_q, n_kv, lens, ring, DEV)


# The context split (ad_plan) picks chunks of 32..1024 positions from the
# span, batch and KV heads; these cases reach chunks of 32 (the first four
# rows) and 64 positions (the window at batch 8), one chunk per sequence
# (spans <= 32 and the group sizes below) and a combine over up to 98
# chunks.
@pytest.mark.parametrize("lens,window,ring", [
    ([3000], 0, 3000),                                   # full context, many chunks
    ([1, 5, 300, 513, 514, 1000, 2000, 4097], 513, 513), # sliding window in a 513-row ring, ragged
    ([17, 100, 64], 0, 100),                             # one chunk per sequence: no combine
    ([700, 129, 128, 127], 513, 600),                    # window with a ring larger than it
    ([1000, 800, 999], 0, 1000),
    ([31, 7, 32], 0, 32),                                # one chunk per sequence
])
def test_flint_heads(lens, window, ring):
    case = _case(31, 32, 4, lens, ring)
    out, err = _run(case, 32, 4, window)
    assert err == 0
    ref, mix = _oracle(case, window)
    _check(out, ref, mix)


@pytest.mark.parametrize("n_q,n_kv", [(4, 4), (16, 1), (24, 8), (12, 4)])
def test_group_sizes(n_q, n_kv):
    case = _case(32, n_q, n_kv, [257, 1, 90], 300)
    out, err = _run(case, n_q, n_kv, 0)
    assert err == 0
    ref, mix = _oracle(case, 0)
    _check(out, ref, mix)


@pytest.mark.parametrize("L", [9000, 20000, 60000, 100000])
def test_long_context_batch1(L):
    """Chunks of 128, 256, 512 and 1024 positions (4 waves of 1, 2, 4, 8
    steps); 100K is the decode context of the pages' measurement."""
    case = _case(33, 32, 4, [L], L)
    out, err = _run(case, 32, 4, 0)
    assert err == 0
    ref, mix = _oracle(case, 0)
    _check(out, ref, mix)


def test_sinks_none_and_dominant():
    case = _case(34, 32, 4, [50, 700], 700)
    case.sinks[:16] = float("-inf")
    case.sinks[16:] = 40.0                  # the sink takes nearly all the weight
    out, err = _run(case, 32, 4, 0)
    assert err == 0
    ref, mix = _oracle(case, 0)
    _check(out, ref, mix)
    assert gen.numpy_f64(out)[:, 16:].max() < 1e-6


def test_invalid_sequences_give_zeros_and_error():
    case = _case(35, 32, 4, [40, 10, 600, 30, 20], 64)
    case.seq_len[1] = 0                     # empty
    case.seq_len[2] = 600                   # full-context span beyond the ring
    case.seq_base[4] = case.n_rows - 10     # ring past the cache
    for max_len in (2000, 600, 64):         # many chunks / one chunk (64: then 600 > max_len too)
        out, err = _run(case, 32, 4, 0, max_len=max_len)
        assert err == 1
        got = gen.numpy_f64(out)
        assert (got[[1, 2, 4]] == 0).all()
        ref, mix = _oracle(gen.DecodeAttnCase(case.q[[0, 3]], case.k_cache, case.v_cache, case.seq_base[[0, 3]],
                                              case.seq_len[[0, 3]], case.sinks, case.ring, case.n_rows), 0)
        _check(out[[0, 3]], ref, mix)


def test_window_longer_than_context_is_full_context():
    case = _case(36, 32, 4, [300, 77], 300)
    a, _ = _run(case, 32, 4, 0)
    b, _ = _run(case, 32, 4, 5000)
    assert torch.equal(a, b)


def test_reproducible():
    case = _case(37, 32, 4, [5000, 3], 5000)
    a, _ = _run(case, 32, 4, 0)
    b, _ = _run(case, 32, 4, 0)
    assert torch.equal(a, b)
