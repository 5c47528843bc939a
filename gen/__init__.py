"""Seeded synthetic inputs for the Flint-shaped W4A16 MoE layer.

This module is shared by the tests, the benchmark and the smoke check, and it
is the ONLY code the CPU oracle (``oracle/``) and the HIP path have in common.
It holds random draws and their arrangement into the source NVFP4 storage
layout, and nothing of the layer's arithmetic: no decoding, no GEMV, no
routing, no rounding beyond torch's own dtype casts of the drawn values.

Value distributions (the input recipe; sizes follow the Flint MoE layer that
"Day-0 Support for Flint on vLLM", section "Model architecture", describes:
hidden 2048, 256 routed experts, sigmoid top-6 and one shared expert):

* router weights   W_r = BF16(N(0, 0.02^2)), shape [E][H]
* E2M1 code bytes  uniform over 0..255 (each nibble uniform over all 16 codes)
* UE4M3 scales     byte (e << 3), e uniform over {3..9}: powers of two 2^-4..2^2
                   ("pow2");  "full" draws e in {3..8} and a uniform 3-bit
                   mantissa, to cover every mantissa decode path
* FP32 scale       1/64 per matrix per expert ("pow2"); "varied" draws a
                   non-power-of-two value in [0.01, 0.03) per matrix
* activations      x = BF16(N(0,1)); "correlated" tokens share a common
                   direction, x_t = BF16(0.6 c + 0.8 z_t), which skews routing
* RMSNorm gamma    BF16(1 + 0.1 N(0,1))

Source NVFP4 layout (the storage the load-time repack reads): a matrix of
R x C values is R rows of C/64 super-blocks of 36 bytes; a super-block holds
4 sub-blocks of 16 values, each one UE4M3 scale byte plus 8 code bytes
(two E2M1 codes per byte).  Byte positions of the four scale bytes:

* "interleaved":  scale of sub-block j at byte 9j, its codes at 9j+1..9j+8
* "scales_first": the four scales at bytes 0..3, the codes at 4..35
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np
import torch

SRC_LAYOUTS = ("interleaved", "scales_first")
SUPERBLOCK_BYTES = 36
SUPERBLOCK_VALUES = 64


@dataclasses.dataclass(frozen=True)
class MoeShape:
    """Sizes of one MoE layer: hidden H, routed experts E, expert
    intermediate I, shared-expert intermediate SI (0 = no shared expert),
    top-k K."""

    hidden: int
    n_experts: int
    inter: int
    shared_inter: int
    top_k: int


# Tiny layer (fits in cache; latency and correctness only).
SHAPE_TINY = MoeShape(hidden=512, n_experts=32, inter=128, shared_inter=128, top_k=4)
# Flint-shaped layer; expert intermediate 512 is an assumption (the pages do
# not print it).
SHAPE_FLINT = MoeShape(hidden=2048, n_experts=256, inter=512, shared_inter=512, top_k=6)
# Dense SwiGLU MLP intermediate of the two dense layers (assumed).
DENSE_INTER = 5632


def seed_for(base: int, *keys) -> int:
    """Deterministic 63-bit seed from a base seed and any hashable labels."""
    h = hashlib.sha256(repr((int(base),) + tuple(keys)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def router_weights(seed: int, n_experts: int, hidden: int, device="cpu") -> torch.Tensor:
    """BF16 router matrix [E][H], entries BF16(N(0, 0.02^2))."""
    g = _gen(seed, device)
    w = torch.randn((n_experts, hidden), generator=g, device=device, dtype=torch.float32)
    return (w * 0.02).to(torch.bfloat16)


def activations(seed: int, batch: int, hidden: int, device="cpu", kind: str = "iid") -> torch.Tensor:
    """BF16 hidden vectors [B][H] ~ N(0,1); kind "correlated" mixes in one
    shared direction so that tokens prefer the same experts."""
    g = _gen(seed, device)
    z = torch.randn((batch, hidden), generator=g, device=device, dtype=torch.float32)
    if kind == "iid":
        return z.to(torch.bfloat16)
    if kind == "correlated":
        c = torch.randn((1, hidden), generator=g, device=device, dtype=torch.float32)
        return (0.6 * c + 0.8 * z).to(torch.bfloat16)
    raise ValueError(f"unknown activation kind {kind!r}")


def rmsnorm_gamma(seed: int, hidden: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    z = torch.randn((hidden,), generator=g, device=device, dtype=torch.float32)
    return (1.0 + 0.1 * z).to(torch.bfloat16)


def _scale_byte_positions(layout: str):
    if layout == "interleaved":
        return [0, 9, 18, 27]
    if layout == "scales_first":
        return [0, 1, 2, 3]
    raise ValueError(f"unknown source layout {layout!r}")


def nvfp4_source(seed: int, n_mats: int, rows: int, cols: int, device="cpu",
                 layout: str = "interleaved", scale_mode: str = "pow2") -> torch.Tensor:
    """Random source super-blocks, uint8 [n_mats][rows][cols/64][36].

    Code bytes are uniform; the four scale bytes of each super-block are
    drawn per ``scale_mode`` ("pow2", "full" or "bytes" = any byte value,
    NaN and sign bit included, for lossless-repack tests)."""
    if cols % SUPERBLOCK_VALUES:
        raise ValueError("cols must be a multiple of 64")
    g = _gen(seed, device)
    nb = cols // SUPERBLOCK_VALUES
    out = torch.randint(0, 256, (n_mats, rows, nb, SUPERBLOCK_BYTES), generator=g,
                        device=device, dtype=torch.uint8)
    if scale_mode == "bytes":
        return out
    shape = (n_mats, rows, nb, 4)
    if scale_mode == "pow2":
        e = torch.randint(3, 10, shape, generator=g, device=device, dtype=torch.uint8)
        sc = e << 3
    elif scale_mode == "full":
        e = torch.randint(3, 9, shape, generator=g, device=device, dtype=torch.uint8)
        m = torch.randint(0, 8, shape, generator=g, device=device, dtype=torch.uint8)
        sc = (e << 3) | m
    else:
        raise ValueError(f"unknown scale mode {scale_mode!r}")
    pos = _scale_byte_positions(layout)
    out[..., pos] = sc
    return out


def tensor_scales(seed: int, n: int, mode: str = "pow2") -> torch.Tensor:
    """FP32 per-tensor scales [n][3] (gate, up, down) on the CPU."""
    if mode == "pow2":
        return torch.full((n, 3), 1.0 / 64.0, dtype=torch.float32)
    if mode == "varied":
        g = _gen(seed, "cpu")
        return 0.01 + 0.02 * torch.rand((n, 3), generator=g, dtype=torch.float32)
    raise ValueError(f"unknown tensor-scale mode {mode!r}")


@dataclasses.dataclass
class MoeLayerSource:
    """One MoE layer in the source storage format (all torch tensors).

    gate, up: uint8 [E][I][H/64][36];  down: uint8 [E][H][I/64][36]
    sh_gate, sh_up: uint8 [1][SI][H/64][36]; sh_down: uint8 [1][H][SI/64][36]
    router: bf16 [E][H];  gscale: f32 [E][3];  sh_gscale: f32 [1][3]
    """

    shape: MoeShape
    layout: str
    router: torch.Tensor
    gate: torch.Tensor
    up: torch.Tensor
    down: torch.Tensor
    sh_gate: torch.Tensor | None
    sh_up: torch.Tensor | None
    sh_down: torch.Tensor | None
    gscale: torch.Tensor
    sh_gscale: torch.Tensor


def moe_layer_source(shape: MoeShape, seed: int, device="cpu", layout: str = "interleaved",
                     scale_mode: str = "pow2", gscale_mode: str = "pow2") -> MoeLayerSource:
    H, E, I, SI = shape.hidden, shape.n_experts, shape.inter, shape.shared_inter
    mk = lambda tid, n, r, c: nvfp4_source(seed_for(seed, tid), n, r, c, device, layout, scale_mode)
    gs = tensor_scales(seed_for(seed, "gscale"), E + 1, gscale_mode)
    return MoeLayerSource(
        shape=shape, layout=layout,
        router=router_weights(seed_for(seed, "router"), E, H, device),
        gate=mk("gate", E, I, H), up=mk("up", E, I, H), down=mk("down", E, H, I),
        sh_gate=mk("sh_gate", 1, SI, H) if SI else None,
        sh_up=mk("sh_up", 1, SI, H) if SI else None,
        sh_down=mk("sh_down", 1, H, SI) if SI else None,
        gscale=gs[:E].contiguous(), sh_gscale=gs[E:].contiguous(),
    )


def dense_mlp_source(hidden: int, inter: int, seed: int, device="cpu", layout: str = "interleaved",
                     scale_mode: str = "pow2", gscale_mode: str = "pow2"):
    """Dense SwiGLU MLP in source format: (gate [1][I][H/64][36], up, down
    [1][H][I/64][36], gscale f32 [1][3])."""
    mk = lambda tid, r, c: nvfp4_source(seed_for(seed, tid), 1, r, c, device, layout, scale_mode)
    return (mk("gate", inter, hidden), mk("up", inter, hidden), mk("down", hidden, inter),
            tensor_scales(seed_for(seed, "gscale"), 1, gscale_mode))


# ------------------------------------------------------------- attention --

@dataclasses.dataclass(frozen=True)
class AttnShape:
    n_q_heads: int
    n_kv_heads: int
    head_dim: int = 128


ATTN_FLINT = AttnShape(n_q_heads=32, n_kv_heads=4, head_dim=128)   # GQA 32/4, d 128


def rope_table(n_pos: int, head_dim: int = 128, base: float = 10000.0, device="cpu") -> torch.Tensor:
    """A caller's rotary table, float32 [n_pos][head_dim]: row p holds the
    cosines of the head_dim / 2 angles p * base^(-2i / head_dim), then their
    sines (angles and functions in float64, stored as float32)."""
    i = torch.arange(head_dim // 2, dtype=torch.float64)
    inv = base ** (-2.0 * i / head_dim)
    ang = torch.arange(n_pos, dtype=torch.float64)[:, None] * inv[None, :]
    return torch.cat([torch.cos(ang), torch.sin(ang)], dim=1).to(torch.float32).to(device)


def attn_rows(seed: int, n_tokens: int, shape: AttnShape, device="cpu") -> torch.Tensor:
    """Projection rows [T][(n_q + 2 n_kv) d] BF16 ~ N(0,1), heads with
    per-head scales spread over two decades so that the norms matter."""
    g = _gen(seed, device)
    n_heads = shape.n_q_heads + 2 * shape.n_kv_heads
    z = torch.randn((n_tokens, n_heads, shape.head_dim), generator=g, device=device, dtype=torch.float32)
    sc = 10.0 ** (2.0 * torch.rand((n_tokens, n_heads, 1), generator=g, device=device) - 1.0)
    return (z * sc).reshape(n_tokens, -1).to(torch.bfloat16)


@dataclasses.dataclass
class DecodeAttnCase:
    q: torch.Tensor          # [B][n_q][d] BF16
    k_cache: torch.Tensor    # [n_rows][n_kv][d] BF16
    v_cache: torch.Tensor
    seq_base: torch.Tensor   # [B] int32
    seq_len: torch.Tensor    # [B] int32
    sinks: torch.Tensor      # [n_q] float32
    ring: int
    n_rows: int


def decode_attn_case(seed: int, n_q: int, n_kv: int, lens, ring: int, device="cpu", d: int = 128,
                     gap: int = 3) -> DecodeAttnCase:
    """One decode query per sequence over a BF16 KV cache: sequence b owns
    rows b (ring + gap) .. + ring - 1 (gap rows between sequences that no
    sequence reads); every row of the cache, read or not, holds draws.
    Queries ~ N(0, 2^2) (after their norm and RoPE the heads are O(1) with
    gamma near 1; the factor makes the softmax peaky), K and V ~ N(0, 1),
    sinks ~ N(0, 2^2)."""
    g = _gen(seed, device)
    B = len(lens)
    n_rows = B * (ring + gap)
    q = (2.0 * torch.randn((B, n_q, d), generator=g, device=device)).to(torch.bfloat16)
    k = torch.randn((n_rows, n_kv, d), generator=g, device=device).to(torch.bfloat16)
    v = torch.randn((n_rows, n_kv, d), generator=g, device=device).to(torch.bfloat16)
    sinks = 2.0 * torch.randn((n_q,), generator=g, device=device)
    base = torch.arange(B, dtype=torch.int32, device=device) * (ring + gap)
    lens_t = torch.tensor(list(lens), dtype=torch.int32, device=device)
    return DecodeAttnCase(q, k, v, base, lens_t, sinks.to(torch.float32), ring, n_rows)


def numpy_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").numpy()


def numpy_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16/f32 tensor to float64."""
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)
