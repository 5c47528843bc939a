"""Pins of the oracle's format layer (CPU only).

Each test ties an oracle function to something other than itself: a golden
fixture derived by hand, the OCP MX table, or a library conversion routine.
"""
import math
import os

import numpy as np
import pytest
import torch

import gen
from oracle import bf16, formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split("#")[0].strip() for ln in f if ln.split("#")[0].strip()]


def test_e2m1_matches_ocp_table():
    rows = [ln.split() for ln in _read("e2m1_values.txt")]
    assert len(rows) == 16
    for code, val in rows:
        got = formats.e2m1_value(int(code))
        want = float(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)
    np.testing.assert_array_equal(formats.E2M1_TABLE, [float(v) for _, v in rows])


def test_ue4m3_matches_torch_float8_e4m3fn_all_bytes():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = formats.UE4M3_TABLE
    assert np.array_equal(np.isnan(lib), np.isnan(ours))
    ok = ~np.isnan(lib)
    np.testing.assert_array_equal(ours[ok], lib[ok])
    np.testing.assert_array_equal(np.signbit(ours[ok]), np.signbit(lib[ok]))
    # the scale values the generator draws: exactly 2^-4 .. 2^2
    assert [formats.ue4m3_value(e << 3) for e in range(3, 10)] == [2.0 ** k for k in range(-4, 3)]


def _golden_superblocks():
    sections, cur = {}, None
    for ln in _read("superblock_handmade.txt"):
        if ln.startswith("["):
            cur = ln.strip("[]")
            sections[cur] = []
        else:
            sections[cur].append(ln.split())
    vals = np.array([float(v) for row in sections.pop("values") for v in row])
    blocks = {k: np.array([[int(b, 16) for b in row] for row in v], dtype=np.uint8)
              for k, v in sections.items()}
    return blocks, vals


@pytest.mark.parametrize("layout", gen.SRC_LAYOUTS)
def test_source_decode_handmade_blocks(layout):
    blocks, want = _golden_superblocks()
    got = formats.decode_source_matrix(blocks[layout][None], layout)[0]
    assert got.shape == (128,)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_source_decode_tensor_scale_and_layout_agreement():
    # the same random logical blocks in both byte orders decode identically,
    # and the per-tensor scale multiplies every value
    rng = np.random.default_rng(3)
    scales = rng.integers(0, 256, (5, 2, 4), dtype=np.uint8)
    codes = rng.integers(0, 256, (5, 2, 4, 8), dtype=np.uint8)
    inter = np.zeros((5, 2, 36), np.uint8)
    first = np.zeros((5, 2, 36), np.uint8)
    for j in range(4):
        inter[..., 9 * j] = scales[..., j]
        inter[..., 9 * j + 1: 9 * j + 9] = codes[..., j, :]
        first[..., j] = scales[..., j]
        first[..., 4 + 8 * j: 12 + 8 * j] = codes[..., j, :]
    a = formats.decode_source_matrix(inter, "interleaved", 0.25)
    b = formats.decode_source_matrix(first, "scales_first", 0.25)
    np.testing.assert_array_equal(np.isnan(a), np.isnan(b))
    np.testing.assert_array_equal(np.nan_to_num(a), np.nan_to_num(b))
    c = formats.decode_source_matrix(inter, "interleaved", 1.0)
    np.testing.assert_array_equal(np.nan_to_num(a), np.nan_to_num(c) * 0.25)
    # element (r, 16j + 2i) is the low nibble of code byte i of sub-block j
    r, blk, j, i = 3, 1, 2, 5
    byte = codes[r, blk, j, i]
    s = formats.UE4M3_TABLE[scales[r, blk, j]]
    col = 64 * blk + 16 * j + 2 * i
    for off, nib in ((0, byte & 15), (1, byte >> 4)):
        want = formats.E2M1_TABLE[nib] * s
        got = c[r, col + off]
        assert (np.isnan(want) and np.isnan(got)) or got == want


def test_bf16_golden_cases():
    for ln in _read("bf16_rounding.txt"):
        src, want = ln.split()[:2]
        x = float.fromhex(src)
        w = float(want) if "inf" in want else float.fromhex(want)
        got = float(bf16.round_bf16(np.array([x]))[0])
        assert got == w and math.copysign(1, got) == math.copysign(1, w), (src, got, w)


def test_bf16_matches_torch_on_float32_values():
    # torch's float32 -> bfloat16 cast rounds to nearest even; on values that
    # float32 holds exactly the direct float64 rounding must agree bit for bit
    g = torch.Generator().manual_seed(0)
    bits = torch.randint(0, 2 ** 31, (200000,), generator=g, dtype=torch.int64)
    bits = bits | (torch.randint(0, 2, (200000,), generator=g) << 31)
    f32 = bits.to(torch.int32).view(torch.float32)
    f32 = f32[torch.isfinite(f32)]
    ties = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 2 ** -130 * 1.5, 3.0e38, -7.0e-39],
                        dtype=torch.float32)
    f32 = torch.cat([f32, ties])
    lib = f32.to(torch.bfloat16).to(torch.float64).numpy()
    ours = bf16.round_bf16(f32.to(torch.float64).numpy())
    np.testing.assert_array_equal(ours, lib)
    np.testing.assert_array_equal(np.signbit(ours), np.signbit(lib))


def test_bf16_nan_and_idempotent():
    x = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1.5])
    y = bf16.round_bf16(x)
    assert np.isnan(y[0]) and y[1] == np.inf and y[2] == -np.inf
    assert np.signbit(y[4]) and y[5] == 1.5
    r = np.random.default_rng(1).standard_normal(1000) * 1e3
    once = bf16.round_bf16(r)
    np.testing.assert_array_equal(bf16.round_bf16(once), once)
