"""float64 -> bfloat16 rounding (oracle).

TEST INFRASTRUCTURE: see the package docstring for who may use it.

bfloat16 keeps float32's 8-bit exponent and 8 significant bits.  The pages
say every Flint kernel rounds where the reference implementation rounds
("Day-0 Support for Flint on vLLM", sections "Model architecture" and
"Optimizations", the norm/SiLU bullet) without listing the points; the
oracle reads "round" as IEEE round-to-nearest-even into bfloat16, applied
directly to the float64 value (no intermediate float32 step, which would
round twice).
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float.fromhex("0x1.fe00000000000p+127")   # largest finite bf16
_MIN_NORMAL_EXP = -125   # frexp exponent of 2^-126, the smallest normal


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even); returns
    float64 holding bf16 values.  Subnormals keep a fixed spacing of 2^-133;
    magnitudes that round above BF16_MAX become infinities; NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0.0)
    xf = x[finite]
    _, e = np.frexp(xf)                       # xf = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, _MIN_NORMAL_EXP)        # below 2^-126 the spacing is fixed
    spacing = np.ldexp(1.0, e - 8)            # 8 significant bits
    q = np.round(xf / spacing) * spacing      # np.round: half to even; the
    q = np.where(np.abs(q) > BF16_MAX, np.copysign(np.inf, q), q)  # scaling is exact
    out[finite] = q
    return out

