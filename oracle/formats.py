"""NVFP4 value definitions and the source super-block decode (oracle).

TEST INFRASTRUCTURE: see the package docstring for who may use it.

Format facts from the pages:
  * arex-research, "vLLM 宣布首日支持 Recursive 的 Flint", section
    "七个内核的依赖链：低延迟路径、无损重排与参考舍入", second paragraph:
    the checkpoint stores NVFP4 as 64-value super-blocks, each four groups of
    one UE4M3 scale and 16 E2M1 codes; there is one FP32 scale per tensor,
    and MoE weights carry theirs per expert.
  * "Day-0 Support for Flint on vLLM", section "Model architecture", the
    paragraph after the bullets: the GGUF blocks are NVFP4 in another byte
    order, repacked losslessly at load.

Readings (the pages do not print them):
  * E2M1 is the 4-bit float of the OCP Microscaling (MX) specification:
    bit 3 sign, bits 2..1 exponent with bias 1, bit 0 mantissa; exponent 0
    is subnormal (0.5 * m).
  * UE4M3 is decoded as E4M3FN (bias 7, subnormals, 0x7F/0xFF = NaN, no
    infinities).  Valid scales have bit 7 clear; the decode still honours it
    as a sign so that every byte has a defined value.
  * Byte order inside the 36-byte super-block: "interleaved" (scale of
    sub-block j at byte 9j, its 16 codes in bytes 9j+1..9j+8) or
    "scales_first" (scales at bytes 0..3, codes at 4..35).  Within a code
    byte, the even element is the low nibble.  Blocks run along the input
    (reduction) dimension of a row-major matrix.
"""
from __future__ import annotations

import math

import numpy as np


def e2m1_value(code: int) -> float:
    """Value of one 4-bit E2M1 code (0..15), from its sign/exponent/mantissa
    fields."""
    code = int(code)
    if not 0 <= code < 16:
        raise ValueError("E2M1 code out of range")
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        mag = 0.5 * man                      # subnormal: 2^(1-bias) * m/2
    else:
        mag = 2.0 ** (exp - 1) * (1.0 + 0.5 * man)
    return sign * mag


def ue4m3_value(byte: int) -> float:
    """Value of one UE4M3 scale byte, decoded with E4M3FN semantics."""
    byte = int(byte)
    if not 0 <= byte < 256:
        raise ValueError("scale byte out of range")
    sign = -1.0 if byte & 0x80 else 1.0
    exp = (byte >> 3) & 0xF
    man = byte & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        mag = 2.0 ** -6 * (man / 8.0)       # subnormal
    else:
        mag = 2.0 ** (exp - 7) * (1.0 + man / 8.0)
    return sign * mag


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
UE4M3_TABLE = np.array([ue4m3_value(b) for b in range(256)], dtype=np.float64)


def split_superblocks(blocks: np.ndarray, layout: str = "interleaved"):
    """Separate source super-blocks [..., 36] into scale bytes [..., 4] and
    code bytes [..., 4, 8] (sub-block j's 8 code bytes in row j)."""
    blocks = np.asarray(blocks, dtype=np.uint8)
    if blocks.shape[-1] != 36:
        raise ValueError("super-blocks must be 36 bytes")
    if layout == "interleaved":
        scales = blocks[..., [0, 9, 18, 27]]
        codes = np.stack([blocks[..., 9 * j + 1: 9 * j + 9] for j in range(4)], axis=-2)
    elif layout == "scales_first":
        scales = blocks[..., 0:4]
        codes = blocks[..., 4:36].reshape(blocks.shape[:-1] + (4, 8))
    else:
        raise ValueError(f"unknown source layout {layout!r}")
    return scales, codes


def decode_source_matrix(blocks: np.ndarray, layout: str = "interleaved",
                         tensor_scale: float = 1.0) -> np.ndarray:
    """Dequantise one source matrix.

    blocks: uint8 [R][C/64][36].  Returns float64 [R][C] with
    W[r, c] = E2M1(code) * UE4M3(scale of c's 16-value group) * tensor_scale,
    every product exact in float64.
    """
    blocks = np.asarray(blocks, dtype=np.uint8)
    if blocks.ndim != 3:
        raise ValueError("expected [rows][cols/64][36]")
    rows, nb, _ = blocks.shape
    scales, codes = split_superblocks(blocks, layout)          # [R,nb,4], [R,nb,4,8]
    lo = codes & 0x0F                                           # even elements
    hi = codes >> 4                                             # odd elements
    nib = np.stack([lo, hi], axis=-1).reshape(rows, nb, 4, 16)  # element 2i, 2i+1
    vals = E2M1_TABLE[nib] * UE4M3_TABLE[scales][..., None]
    return vals.reshape(rows, nb * 64) * float(tensor_scale)
