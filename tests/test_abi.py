"""The C-ABI library loads on the CPU, exports every symbol the header
declares, and rejects bad arguments before enqueuing anything (these checks
make no HIP call, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

import w4a16_moe_decode_amd as fm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flint_moe.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^FLINT_API\s+[\w\s\*]+?\b(flint_\w+)\s*\(", src, re.M)))


def test_header_declarations_match_binding_list():
    assert _declared() == sorted(fm.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = fm.lib()
    for name in _declared():
        assert hasattr(L, name), name
    # nothing but the C ABI is exported
    out = os.popen(f"nm -D --defined-only {fm.LIB_PATH}").read()
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert exported == set(_declared())


def test_version_and_status_strings():
    assert fm.version().startswith("flint-moe")
    assert fm.status_string(fm.FLINT_OK) == "ok"
    assert fm.status_string(fm.FLINT_ERR_UNSUPPORTED).startswith("unsupported")
    assert fm.status_string(12345) == "unknown"


def test_packed_and_workspace_sizes():
    assert fm.flint_nvfp4_packed_bytes(2, 512, 2048) == (2 * 512 * 1024, 2 * 512 * 128)
    with pytest.raises(fm.FlintError):
        fm.flint_nvfp4_packed_bytes(1, 4, 100)          # cols not a multiple of 64
    s = fm.FlintMoeShape(2048, 256, 512, 512, 6, 0, 1e-6)
    ws = fm.flint_moe_workspace_bytes(s, 8)
    # at least the h buffer: (min(8*6, 256) + 1) slots x 8 tokens x 512 x 2 bytes
    assert ws >= 49 * 8 * 512 * 2
    # decode needs the same layout for any batch; prefill grows with tokens
    assert fm.flint_moe_workspace_bytes(s, 1) <= ws
    assert fm.flint_moe_workspace_bytes(s, 8192) > 8192 * 6 * 2048 * 4
    bad = fm.FlintMoeShape(2048, 256, 500, 512, 6, 0, 1e-6)
    assert fm.lib().flint_moe_workspace_bytes(ctypes.byref(bad), 1) == -fm.FLINT_ERR_UNSUPPORTED


def _decode_status(shape, weights, x=16, batch=1, out=32, ws=1024, ws_bytes=1 << 30, gamma=None):
    L = fm.lib()
    v = lambda a: None if a is None else ctypes.c_void_p(a)
    return L.flint_moe_decode(ctypes.byref(shape), ctypes.byref(weights), v(x), batch, v(out), None,
                              None, v(gamma), v(ws), ws_bytes, None)


def _fake_weights(align=16):
    w = fm.FlintMoeWeights()
    for i, (f, _) in enumerate(fm.FlintMoeWeights._fields_):
        setattr(w, f, 4096 * (i + 1) + (0 if align == 16 else 4))
    return w


def test_decode_validation_codes():
    s = fm.FlintMoeShape(2048, 256, 512, 512, 6, 0, 1e-6)
    w = _fake_weights()
    assert _decode_status(s, w, batch=9) == fm.FLINT_ERR_UNSUPPORTED     # use prefill
    assert _decode_status(s, w, batch=0) == fm.FLINT_ERR_INVALID_ARG
    assert _decode_status(s, w, x=None) == fm.FLINT_ERR_INVALID_ARG
    assert _decode_status(s, w, x=20) == fm.FLINT_ERR_ALIGNMENT
    assert _decode_status(s, w, ws=None) == fm.FLINT_ERR_WORKSPACE
    assert _decode_status(s, w, ws_bytes=100) == fm.FLINT_ERR_WORKSPACE
    assert _decode_status(s, w, out=16) == fm.FLINT_ERR_INVALID_ARG     # out == x without residual
    assert _decode_status(s, _fake_weights(align=4)) == fm.FLINT_ERR_ALIGNMENT
    w2 = _fake_weights()
    w2.d_codes = None
    assert _decode_status(s, w2) == fm.FLINT_ERR_INVALID_ARG
    for bad in (fm.FlintMoeShape(2048, 256, 512, 512, 9, 0, 1e-6),      # top_k > 8
                fm.FlintMoeShape(2048, 257, 512, 512, 6, 0, 1e-6),      # > 256 experts
                fm.FlintMoeShape(2000, 256, 512, 512, 6, 0, 1e-6),      # H not a multiple of 64
                fm.FlintMoeShape(2048, 4, 512, 512, 6, 0, 1e-6),        # top_k > E
                fm.FlintMoeShape(2048, 256, 512, 512, 6, 0x100, 1e-6)):  # unknown flag
        assert _decode_status(bad, w) == fm.FLINT_ERR_UNSUPPORTED
    L = fm.lib()
    v = ctypes.c_void_p
    for idx_ptr, want in ((v(4100), fm.FLINT_OK), (v(4098), fm.FLINT_ERR_ALIGNMENT)):
        # top-k outputs need 4-byte alignment only; validation order puts the
        # workspace check last, so a good pointer reaches FLINT_ERR_WORKSPACE
        st = L.flint_moe_decode(ctypes.byref(s), ctypes.byref(w), v(16), 1, v(32), idx_ptr, None,
                                None, v(1024), 10, None)
        assert st == (fm.FLINT_ERR_WORKSPACE if want == fm.FLINT_OK else want)
    pre = fm.FlintMoeShape(2048, 256, 512, 512, 6, fm.FLINT_PRE_RMSNORM, 1e-6)
    assert _decode_status(pre, w, gamma=None) == fm.FLINT_ERR_INVALID_ARG
    L = fm.lib()
    assert L.flint_moe_decode_stage(3, ctypes.byref(s), ctypes.byref(w), ctypes.c_void_p(16), 1,
                                    ctypes.c_void_p(32), None, None, None, ctypes.c_void_p(1024),
                                    1 << 30, None) == fm.FLINT_ERR_INVALID_ARG


def test_repack_and_dense_validation_codes():
    L = fm.lib()
    v = ctypes.c_void_p
    assert L.flint_moe_repack(v(16), 1, 4, 96, 0, v(32), v(48), 1, None) == fm.FLINT_ERR_UNSUPPORTED
    assert L.flint_moe_repack(v(16), 1, 4, 64, 7, v(32), v(48), 1, None) == fm.FLINT_ERR_UNSUPPORTED
    assert L.flint_moe_repack(None, 1, 4, 64, 0, v(32), v(48), 1, None) == fm.FLINT_ERR_INVALID_ARG
    assert L.flint_moe_repack(v(18), 1, 4, 64, 0, v(32), v(48), 1, None) == fm.FLINT_ERR_ALIGNMENT
    assert L.flint_moe_unpack(v(16), v(32), 0, 4, 64, 0, 1, v(48), None) == fm.FLINT_ERR_INVALID_ARG
    d = L.flint_dense_gemv
    eps = ctypes.c_float(1e-6)
    assert d(v(16), v(32), v(48), None, 64, 64, 0, v(64), 9, v(80), 0, None, None, eps, None) \
        == fm.FLINT_ERR_UNSUPPORTED
    assert d(v(16), v(32), v(48), None, 64, 64, 0, v(64), 1, v(80), 5, None, None, eps, None) \
        == fm.FLINT_ERR_UNSUPPORTED
    assert d(v(16), v(32), v(48), None, 64, 64, 0, v(64), 1, v(80), fm.FLINT_EPI_RESIDUAL, None,
             None, eps, None) == fm.FLINT_ERR_INVALID_ARG
    assert d(v(16), v(32), v(48), None, 64, 64, fm.FLINT_PRE_RMSNORM, v(64), 1, v(80),
             fm.FLINT_EPI_NONE, None, v(96), eps, None) == fm.FLINT_ERR_UNSUPPORTED
    assert d(None, None, None, None, 64, 64, fm.FLINT_W_BF16, v(64), 1, v(80), 0, None, None, eps,
             None) == fm.FLINT_ERR_INVALID_ARG


def test_decode_path_rules():
    """Which kernels a decode call runs: host logic only, nothing enqueued."""
    flint = fm.FlintMoeShape(2048, 256, 512, 512, 6, 0, 1e-6)
    assert fm.flint_moe_decode_path(flint, 1) == fm.FLINT_PATH_SINGLE_ONE
    for b in range(2, 9):
        assert fm.flint_moe_decode_path(flint, b) == fm.FLINT_PATH_SINGLE_BATCH
    for k in (1, 8):                                # any top-k up to the maximum
        s = fm.FlintMoeShape(2048, 256, 512, 512, k, 0, 1e-6)
        assert fm.flint_moe_decode_path(s, 8) == fm.FLINT_PATH_SINGLE_BATCH
    for other in (fm.FlintMoeShape(2048, 256, 512, 1024, 6, 0, 1e-6),
                  fm.FlintMoeShape(2048, 128, 512, 512, 6, 0, 1e-6),
                  fm.FlintMoeShape(4096, 256, 512, 512, 6, 0, 1e-6)):
        assert fm.flint_moe_decode_path(other, 4) == fm.FLINT_PATH_SPLIT
    # the old single-launch batch flag is no longer accepted
    with pytest.raises(fm.FlintError) as e:
        fm.flint_moe_decode_path(fm.FlintMoeShape(2048, 256, 512, 512, 6, 0x20, 1e-6), 2)
    assert e.value.status == fm.FLINT_ERR_UNSUPPORTED
    for flags in (fm.FLINT_SPLIT, fm.FLINT_W_BF16):
        s = fm.FlintMoeShape(2048, 256, 512, 512, 6, flags, 1e-6)
        # W16A16 at batch 1 takes the BF16 form of the single launch
        want1 = fm.FLINT_PATH_SINGLE_ONE if flags == fm.FLINT_W_BF16 else fm.FLINT_PATH_SPLIT
        assert fm.flint_moe_decode_path(s, 1) == want1
        assert fm.flint_moe_decode_path(s, 8) == fm.FLINT_PATH_SPLIT
    tiny = fm.FlintMoeShape(512, 32, 128, 128, 4, 0, 1e-6)          # hidden not a multiple of 2048
    assert fm.flint_moe_decode_path(tiny, 1) == fm.FLINT_PATH_SPLIT
    wide = fm.FlintMoeShape(2048, 48, 512, 1024, 8, 0, 1e-6)
    assert fm.flint_moe_decode_path(wide, 1) == fm.FLINT_PATH_SINGLE_ONE
    assert fm.flint_moe_decode_path(wide, 3) == fm.FLINT_PATH_SPLIT
    for b in (0, 9):
        with pytest.raises(fm.FlintError) as e:
            fm.flint_moe_decode_path(flint, b)
        assert e.value.status == fm.FLINT_ERR_UNSUPPORTED
    with pytest.raises(fm.FlintError) as e:
        fm.flint_moe_decode_path(fm.FlintMoeShape(2048, 256, 512, 512, 0, 0, 1e-6), 1)
    assert e.value.status == fm.FLINT_ERR_INVALID_ARG


def test_decode_stack_validation_codes():
    """flint_moe_decode_stack rejects bad arguments before enqueuing anything
    (fake device addresses: nothing is dereferenced on the host)."""
    L = fm.lib()
    v = ctypes.c_void_p
    s = fm.FlintMoeShape(2048, 256, 512, 512, 6, 0, 1e-6)
    big = 1 << 40

    def st(shape=s, layers=v(64), n=3, gam=v(128), x=v(256), out=v(256), idx=v(512), w=v(768),
           lo=None, ws=None, ws_bytes=big):
        return L.flint_moe_decode_stack(ctypes.byref(shape), layers, n, gam, x, out, idx, w, lo, ws,
                                        ws_bytes, None)

    assert st(n=0) == fm.FLINT_ERR_INVALID_ARG
    assert st(n=5000) == fm.FLINT_ERR_UNSUPPORTED                          # > 4096 layers
    assert st(layers=None) == fm.FLINT_ERR_INVALID_ARG
    assert st(gam=v(130)) == fm.FLINT_ERR_ALIGNMENT
    assert st(idx=None) == fm.FLINT_ERR_INVALID_ARG
    assert st(w=v(770)) == fm.FLINT_ERR_ALIGNMENT
    assert st(lo=v(8)) == fm.FLINT_ERR_ALIGNMENT
    assert st() == fm.FLINT_ERR_WORKSPACE                                  # ws missing
    assert st(ws=v(4096), ws_bytes=100) == fm.FLINT_ERR_WORKSPACE
    for flags in (fm.FLINT_PRE_RMSNORM, fm.FLINT_RESIDUAL, fm.FLINT_W_BF16, fm.FLINT_SPLIT):
        assert st(shape=fm.FlintMoeShape(2048, 256, 512, 512, 6, flags, 1e-6)) == fm.FLINT_ERR_UNSUPPORTED
    # outside the one-token single-launch envelope (hidden 512)
    assert st(shape=fm.FlintMoeShape(512, 32, 128, 128, 4, 0, 1e-6), ws=v(4096)) == fm.FLINT_ERR_UNSUPPORTED


def test_workspace_error_query_validation():
    """flint_moe_workspace_error checks its arguments before enqueuing the
    copy of the header's error word."""
    L = fm.lib()
    v = ctypes.c_void_p
    assert L.flint_moe_workspace_error(None, 4096, v(64), None) == fm.FLINT_ERR_INVALID_ARG
    assert L.flint_moe_workspace_error(v(4096), 4096, None, None) == fm.FLINT_ERR_INVALID_ARG
    assert L.flint_moe_workspace_error(v(4100), 4096, v(64), None) == fm.FLINT_ERR_ALIGNMENT
    assert L.flint_moe_workspace_error(v(4096), 4096, v(66), None) == fm.FLINT_ERR_ALIGNMENT
    assert L.flint_moe_workspace_error(v(4096), 1000, v(64), None) == fm.FLINT_ERR_WORKSPACE
    assert fm.WS_ERROR_OFFSET == 512 and fm.WS_WAIT_LIMIT_OFFSET == 768


def test_decode_and_prefill_workspace_parts_do_not_overlap():
    """The prefill part of a workspace starts after the whole decode part, so
    one workspace serves both kinds of call: the size for T tokens is the
    decode part plus a prefill part that grows with T."""
    s = fm.FlintMoeShape(2048, 256, 512, 512, 6, 0, 1e-6)
    sizes = [fm.flint_moe_workspace_bytes(s, t) for t in (1, 2, 8, 9, 100, 8192)]
    assert sizes == sorted(sizes) and len(set(sizes)) == len(sizes)
    # the decode part alone: a prefill of one token needs more than it
    L = fm.lib()
    v = ctypes.c_void_p
    w = _fake_weights()
    dec_ok = _decode_status(s, w, ws=4096, ws_bytes=sizes[0])
    assert dec_ok != fm.FLINT_ERR_WORKSPACE
    st = L.flint_moe_prefill(ctypes.byref(s), ctypes.byref(w), v(16), 2, v(32), None, None, None,
                             v(4096), sizes[0], None)
    assert st == fm.FLINT_ERR_WORKSPACE                 # 2 tokens need more than the 1-token size


def test_stream_read_validation_codes():
    """The measurement read checks its arguments before enqueuing anything."""
    L = fm.lib()
    v = ctypes.c_void_p
    s = L.flint_stream_read
    assert s(None, 64, 256, 8, 1, v(16), None) == fm.FLINT_ERR_INVALID_ARG
    assert s(v(16), 0, 256, 8, 1, v(16), None) == fm.FLINT_ERR_INVALID_ARG
    assert s(v(16), 24, 256, 8, 1, v(16), None) == fm.FLINT_ERR_INVALID_ARG     # not whole 16-byte words
    assert s(v(16), 64, 256, 8, 0, v(16), None) == fm.FLINT_ERR_INVALID_ARG
    assert s(v(16), 64, 256, 8, 1, None, None) == fm.FLINT_ERR_INVALID_ARG
    assert s(v(24), 64, 256, 8, 1, v(16), None) == fm.FLINT_ERR_ALIGNMENT
    assert s(v(16), 64, 96, 8, 1, v(16), None) == fm.FLINT_ERR_UNSUPPORTED      # threads not 64k
    assert s(v(16), 64, 2048, 8, 1, v(16), None) == fm.FLINT_ERR_UNSUPPORTED
    assert s(v(16), 64, 256, 5, 1, v(16), None) == fm.FLINT_ERR_UNSUPPORTED     # loads not 4/8/16/27


def test_qk_norm_rope_kv_validation_codes():
    """The fused Q/K norm + RoPE + KV write checks its arguments before
    enqueuing anything."""
    L = fm.lib()
    v = ctypes.c_void_p
    f = L.flint_qk_norm_rope_kv
    ok = fm.FlintAttnShape(32, 4, 128, fm.FLINT_ATTN_ROPE, 1e-6)
    nope = fm.FlintAttnShape(32, 4, 128, 0, 1e-6)
    args = lambda sh, **kw: [ctypes.byref(sh), kw.get("qkv", v(16)), kw.get("T", 8), kw.get("pos", v(32)),
                             kw.get("cs", v(48)), kw.get("P", 600), kw.get("slots", v(64)), kw.get("kc", v(80)),
                             kw.get("vc", v(96)), kw.get("S", 100), kw.get("gq", v(112)), kw.get("gk", v(128)),
                             kw.get("q", v(144)), kw.get("err", None), None]
    assert f(*args(ok, qkv=None)) == fm.FLINT_ERR_INVALID_ARG
    assert f(*args(ok, slots=None)) == fm.FLINT_ERR_INVALID_ARG
    assert f(*args(ok, T=0)) == fm.FLINT_ERR_INVALID_ARG
    assert f(*args(ok, S=0)) == fm.FLINT_ERR_INVALID_ARG
    assert f(*args(ok, pos=None)) == fm.FLINT_ERR_INVALID_ARG          # RoPE needs positions and a table
    assert f(*args(ok, cs=None)) == fm.FLINT_ERR_INVALID_ARG
    assert f(*args(ok, P=0)) == fm.FLINT_ERR_INVALID_ARG
    for bad in (fm.FlintAttnShape(32, 4, 64, 0, 1e-6), fm.FlintAttnShape(30, 4, 128, 0, 1e-6),
                fm.FlintAttnShape(32, 4, 128, 0x2, 1e-6), fm.FlintAttnShape(32, 4, 128, 0, -1.0)):
        assert f(*args(bad)) == fm.FLINT_ERR_UNSUPPORTED
    assert f(*args(ok, qkv=v(18))) == fm.FLINT_ERR_ALIGNMENT
    assert f(*args(ok, slots=v(66))) == fm.FLINT_ERR_ALIGNMENT
    assert f(*args(ok, cs=v(52))) == fm.FLINT_ERR_ALIGNMENT
    assert f(*args(ok, err=v(34))) == fm.FLINT_ERR_ALIGNMENT
    # without RoPE the table and positions are not needed (and not checked)
    assert f(*args(nope, qkv=None, pos=None, cs=None, P=0)) == fm.FLINT_ERR_INVALID_ARG


def test_decode_attention_validation_codes():
    """Decode attention checks its arguments before enqueuing anything, and
    sizes its workspace from the shape, window, batch and longest context."""
    L = fm.lib()
    v = ctypes.c_void_p
    f = L.flint_decode_attention
    ok = fm.FlintAttnShape(32, 4, 128, 0, 0.0)
    args = lambda sh, **kw: [ctypes.byref(sh), kw.get("W", 0), kw.get("ring", 1000), kw.get("scale", 0.088),
                             kw.get("q", v(16)), kw.get("B", 1), kw.get("kc", v(32)), kw.get("vc", v(48)),
                             kw.get("rows", 1000), kw.get("base", v(64)), kw.get("len", v(80)),
                             kw.get("max_len", kw.get("ML", 1000)), kw.get("sinks", v(96)), kw.get("out", v(112)),
                             kw.get("ws", v(128)), kw.get("wsb", 1 << 30), kw.get("err", None), None]
    assert f(*args(ok, q=None)) == fm.FLINT_ERR_INVALID_ARG
    assert f(*args(ok, sinks=None)) == fm.FLINT_ERR_INVALID_ARG
    assert f(*args(ok, B=0)) == fm.FLINT_ERR_INVALID_ARG
    assert f(*args(ok, ML=0)) == fm.FLINT_ERR_INVALID_ARG
    assert f(*args(ok, W=-1)) == fm.FLINT_ERR_INVALID_ARG
    assert f(*args(ok, ring=0)) == fm.FLINT_ERR_INVALID_ARG
    assert f(*args(ok, scale=0.0)) == fm.FLINT_ERR_INVALID_ARG
    assert f(*args(ok, scale=float("inf"))) == fm.FLINT_ERR_INVALID_ARG
    assert f(*args(ok, scale=float("nan"))) == fm.FLINT_ERR_INVALID_ARG
    for bad in (fm.FlintAttnShape(32, 4, 64, 0, 0.0), fm.FlintAttnShape(30, 4, 128, 0, 0.0),
                fm.FlintAttnShape(32, 1, 128, 0, 0.0), fm.FlintAttnShape(32, 4, 128, fm.FLINT_ATTN_ROPE, 0.0)):
        assert f(*args(bad)) == fm.FLINT_ERR_UNSUPPORTED               # group > 16, rope flag, head dim
    assert f(*args(ok, rows=1 << 24)) == fm.FLINT_ERR_UNSUPPORTED       # 32-bit element offsets
    assert f(*args(ok, q=v(18))) == fm.FLINT_ERR_ALIGNMENT
    assert f(*args(ok, base=v(66))) == fm.FLINT_ERR_ALIGNMENT
    assert f(*args(ok, err=v(34))) == fm.FLINT_ERR_ALIGNMENT
    wsb = fm.flint_decode_attention_workspace_bytes(ok, 0, 1, 100000)
    assert wsb > 0 and wsb % 16 == 0
    assert f(*args(ok, ML=100000, ring=100000, rows=100000, wsb=wsb - 16)) == fm.FLINT_ERR_WORKSPACE
    assert f(*args(ok, ML=100000, ring=100000, rows=100000, ws=None)) == fm.FLINT_ERR_WORKSPACE
    # one chunk per sequence needs no workspace
    assert fm.flint_decode_attention_workspace_bytes(ok, 513, 1, 32) == 0
    assert fm.flint_decode_attention_workspace_bytes(ok, 513, 8, 100000) > 0
    assert L.flint_decode_attention_workspace_bytes(ctypes.byref(fm.FlintAttnShape(32, 4, 64, 0, 0.0)), 0, 1, 10) < 0


def test_prefill_layout_and_tiled_validation_codes():
    """Argument checks of flint_moe_prefill_layout and flint_moe_prefill_tiled
    (each call fails before any work is queued)."""
    L = fm.lib()
    v = ctypes.c_void_p
    lay = L.flint_moe_prefill_layout
    ok = (v(4096), v(1 << 20), 4, 64, 256, 0, v(1 << 24), v(1 << 28), None)
    assert lay(None, *ok[1:]) == fm.FLINT_ERR_INVALID_ARG
    assert lay(*ok[:6], None, *ok[7:]) == fm.FLINT_ERR_INVALID_ARG
    assert lay(*ok[:2], 0, *ok[3:]) == fm.FLINT_ERR_INVALID_ARG              # no matrices
    assert lay(*ok[:4], 192, *ok[5:]) == fm.FLINT_ERR_INVALID_ARG            # cols not a multiple of 128
    assert lay(*ok[:3], 48, *ok[4:]) == fm.FLINT_ERR_INVALID_ARG             # rows not a multiple of 32
    assert lay(v(4096), v(1 << 20), 3, 16, 256, 1, *ok[6:]) == fm.FLINT_ERR_INVALID_ARG   # odd pair count
    assert lay(*ok[:5], 2, *ok[6:]) == fm.FLINT_ERR_INVALID_ARG              # interleave 0 or 1
    assert lay(v(4100), *ok[1:]) == fm.FLINT_ERR_ALIGNMENT
    assert lay(*ok[:7], v((1 << 28) + 4), None) == fm.FLINT_ERR_ALIGNMENT
    # overlap: 4 x 64 x 256 matrices are 32 KB of codes; outputs starting inside the inputs
    assert lay(v(4096), v(1 << 20), 4, 64, 256, 0, v(4096 + 16384), v(1 << 28), None) == fm.FLINT_ERR_INVALID_ARG
    assert lay(v(4096), v(1 << 20), 4, 64, 256, 0, v(1 << 24), v((1 << 20) + 1024), None) == fm.FLINT_ERR_INVALID_ARG
    # the tiled prefill: a planes struct with a missing or misaligned plane
    s = fm.FlintMoeShape(2048, 256, 512, 512, 6, 0, 1e-6)
    w = _fake_weights()
    ws_bytes = fm.flint_moe_workspace_bytes(s, 16)
    def tiled(planes):
        return L.flint_moe_prefill_tiled(ctypes.byref(s), ctypes.byref(w), ctypes.byref(planes), v(16), 16, v(32),
                                         None, None, None, v(4096), ws_bytes, None)
    full = {f: 1 << (20 + i) for i, (f, _) in enumerate(fm.FlintPrefillPlanes._fields_)}
    for f in full:
        p = fm.FlintPrefillPlanes(**{k: (None if k == f else a) for k, a in full.items()})
        assert tiled(p) == fm.FLINT_ERR_INVALID_ARG, f
        p = fm.FlintPrefillPlanes(**{k: (a + 4 if k == f else a) for k, a in full.items()})
        assert tiled(p) == fm.FLINT_ERR_ALIGNMENT, f
