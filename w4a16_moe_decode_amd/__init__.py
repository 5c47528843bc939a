"""Python binding of libflint_moe.so, the MI355X (gfx950) W4A16 MoE library.

Thin ctypes marshalling over the C ABI in ``include/flint_moe.h``: every
function named ``flint_*`` here calls the C function of the same name with
the data pointers of torch tensors and the current HIP stream.  PyTorch only
provides device memory and streams; all arithmetic of the layer runs in the
library's HIP kernels.  There is no CPU fallback: when the library is not
built, every call raises.

Higher-level helpers (``pack_moe_layer``, ``PackedMoeLayer``) allocate the
packed planes with torch and fill them with ``flint_moe_repack``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

from ._build import LIB_PATH as _DEFAULT_LIB

# FLINT_MOE_LIB names another build of the library to load (the host-sanitizer
# build for CPU-only checks of the C ABI); unset, the in-tree library.
LIB_PATH = os.environ.get("FLINT_MOE_LIB") or _DEFAULT_LIB

# ---------------------------------------------------------------- constants --
FLINT_OK = 0
FLINT_ERR_INVALID_ARG = 1
FLINT_ERR_ALIGNMENT = 2
FLINT_ERR_UNSUPPORTED = 3
FLINT_ERR_WORKSPACE = 4
FLINT_ERR_DEVICE = 5

FLINT_RENORM = 0x1
FLINT_W_BF16 = 0x2
FLINT_PRE_RMSNORM = 0x4
FLINT_RESIDUAL = 0x8
FLINT_SPLIT = 0x10

FLINT_PATH_SPLIT = 0
FLINT_PATH_SINGLE_ONE = 1
FLINT_PATH_SINGLE_BATCH = 2

FLINT_SRC_INTERLEAVED = 0
FLINT_SRC_SCALES_FIRST = 1
SRC_LAYOUT_CODES = {"interleaved": FLINT_SRC_INTERLEAVED, "scales_first": FLINT_SRC_SCALES_FIRST}

FLINT_EPI_NONE = 0
FLINT_EPI_SWIGLU = 1
FLINT_EPI_RESIDUAL = 2

FLINT_ATTN_ROPE = 0x1

MAX_DECODE_BATCH = 8
WS_ERROR_OFFSET = 512
WS_WAIT_LIMIT_OFFSET = 768

# Every symbol the header declares (checked by the CPU export test).
EXPORTS = (
    "flint_version", "flint_status_string", "flint_nvfp4_packed_bytes",
    "flint_moe_workspace_bytes", "flint_moe_workspace_error", "flint_moe_repack", "flint_moe_unpack", "flint_nvfp4_dequant",
    "flint_moe_decode", "flint_moe_decode_noalloc", "flint_moe_decode_stage", "flint_moe_decode_path", "flint_moe_decode_stack",
    "flint_moe_prefill", "flint_moe_prefill_layout", "flint_moe_prefill_tiled", "flint_dense_gemv", "flint_qk_norm_rope_kv", "flint_decode_attention",
    "flint_decode_attention_workspace_bytes", "flint_stream_read",
)


class FlintError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


class FlintMoeShape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("flags", ctypes.c_uint32), ("rms_eps", ctypes.c_float)]


class FlintAttnShape(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("rms_eps", ctypes.c_float)]


class FlintMoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "router", "gu_codes", "gu_scales", "d_codes", "d_scales", "gscale",
        "sh_gu_codes", "sh_gu_scales", "sh_d_codes", "sh_d_scales", "sh_gscale",
        "gu_bf16", "d_bf16", "sh_gu_bf16", "sh_d_bf16")]


class FlintPrefillPlanes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "gu_codes", "gu_scales", "d_codes", "d_scales",
        "sh_gu_codes", "sh_gu_scales", "sh_d_codes", "sh_d_scales")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
        L.flint_version.restype = ctypes.c_char_p
        L.flint_status_string.restype = ctypes.c_char_p
        L.flint_status_string.argtypes = [i32]
        L.flint_nvfp4_packed_bytes.restype = i32
        L.flint_nvfp4_packed_bytes.argtypes = [i64, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.flint_moe_workspace_bytes.restype = i64
        L.flint_moe_workspace_bytes.argtypes = [ctypes.POINTER(FlintMoeShape), i32]
        L.flint_moe_workspace_error.restype = i32
        L.flint_moe_workspace_error.argtypes = [vp, i64, vp, vp]
        L.flint_moe_repack.restype = i32
        L.flint_moe_repack.argtypes = [vp, i64, i32, i32, i32, vp, vp, i64, vp]
        L.flint_moe_unpack.restype = i32
        L.flint_moe_unpack.argtypes = [vp, vp, i64, i32, i32, i32, i64, vp, vp]
        L.flint_nvfp4_dequant.restype = i32
        L.flint_nvfp4_dequant.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp]
        dec = [ctypes.POINTER(FlintMoeShape), ctypes.POINTER(FlintMoeWeights), vp, i32, vp, vp, vp,
               vp, vp, i64, vp]
        L.flint_moe_decode.restype = i32
        L.flint_moe_decode.argtypes = dec
        L.flint_moe_decode_noalloc.restype = i32
        L.flint_moe_decode_noalloc.argtypes = dec[:8] + [vp]
        L.flint_moe_decode_stage.restype = i32
        L.flint_moe_decode_stage.argtypes = [i32] + dec
        L.flint_moe_decode_path.restype = i32
        L.flint_moe_decode_stack.restype = i32
        L.flint_moe_decode_stack.argtypes = [ctypes.POINTER(FlintMoeShape), vp, i32, vp, vp, vp, vp, vp, vp,
                                             vp, i64, vp]
        L.flint_moe_decode_path.argtypes = [ctypes.POINTER(FlintMoeShape), i32]
        L.flint_moe_prefill.restype = i32
        L.flint_moe_prefill.argtypes = dec
        L.flint_moe_prefill_layout.restype = i32
        L.flint_moe_prefill_layout.argtypes = [vp, vp, i64, i32, i32, i32, vp, vp, vp]
        L.flint_moe_prefill_tiled.restype = i32
        L.flint_moe_prefill_tiled.argtypes = dec[:2] + [ctypes.POINTER(FlintPrefillPlanes)] + dec[2:]
        L.flint_dense_gemv.restype = i32
        L.flint_dense_gemv.argtypes = [vp, vp, vp, vp, i32, i32, u32, vp, i32, vp, i32, vp, vp,
                                       ctypes.c_float, vp]
        L.flint_qk_norm_rope_kv.restype = i32
        L.flint_qk_norm_rope_kv.argtypes = [ctypes.POINTER(FlintAttnShape), vp, i32, vp, vp, i32, vp, vp, vp,
                                            i32, vp, vp, vp, vp, vp]
        L.flint_decode_attention_workspace_bytes.restype = i64
        L.flint_decode_attention_workspace_bytes.argtypes = [ctypes.POINTER(FlintAttnShape), i32, i32, i32]
        L.flint_decode_attention.restype = i32
        L.flint_decode_attention.argtypes = [ctypes.POINTER(FlintAttnShape), i32, i32, ctypes.c_float, vp, i32,
                                             vp, vp, i32, vp, vp, i32, vp, vp, vp, i64, vp, vp]
        L.flint_stream_read.restype = i32
        L.flint_stream_read.argtypes = [vp, i64, i32, i32, i32, vp, vp]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().flint_status_string(int(status)).decode()


def version() -> str:
    return lib().flint_version().decode()


def _check(fn: str, status: int):
    if status != FLINT_OK:
        raise FlintError(fn, status)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


# -------------------------------------------------------- raw C-ABI calls --

def flint_nvfp4_packed_bytes(n_mats: int, rows: int, cols: int):
    cb, sb = ctypes.c_int64(), ctypes.c_int64()
    _check("flint_nvfp4_packed_bytes",
           lib().flint_nvfp4_packed_bytes(n_mats, rows, cols, ctypes.byref(cb), ctypes.byref(sb)))
    return cb.value, sb.value


def flint_moe_workspace_bytes(shape: FlintMoeShape, max_tokens: int) -> int:
    v = lib().flint_moe_workspace_bytes(ctypes.byref(shape), int(max_tokens))
    if v < 0:
        raise FlintError("flint_moe_workspace_bytes", -v)
    return v


def flint_moe_workspace_error(ws, ws_bytes, dst, stream=None):
    """Enqueue a copy of the workspace's hand-off error word into ``dst``
    (a device int32/uint32 tensor of at least one element)."""
    _check("flint_moe_workspace_error",
           lib().flint_moe_workspace_error(_p(ws), int(ws_bytes), _p(dst), _stream(stream)))


def flint_moe_repack(src, n_mats, rows, cols, src_layout, dst_codes, dst_scales, dst_mat_stride=1,
                     stream=None):
    _check("flint_moe_repack", lib().flint_moe_repack(
        _p(src), n_mats, rows, cols, src_layout, _p(dst_codes), _p(dst_scales), dst_mat_stride,
        _stream(stream)))


def flint_moe_unpack(codes, scales, n_mats, rows, cols, src_layout, src_mat_stride, dst, stream=None):
    _check("flint_moe_unpack", lib().flint_moe_unpack(
        _p(codes), _p(scales), n_mats, rows, cols, src_layout, src_mat_stride, _p(dst),
        _stream(stream)))


def flint_nvfp4_dequant(codes, scales, n_mats, rows, cols, tensor_scale, out, stream=None):
    _check("flint_nvfp4_dequant", lib().flint_nvfp4_dequant(
        _p(codes), _p(scales), n_mats, rows, cols, _p(tensor_scale), _p(out), _stream(stream)))


def flint_moe_decode(shape, weights, x, batch, out, topk_idx, topk_w, gamma, ws, ws_bytes, stream=None):
    _check("flint_moe_decode", lib().flint_moe_decode(
        ctypes.byref(shape), ctypes.byref(weights), _p(x), batch, _p(out), _p(topk_idx), _p(topk_w),
        _p(gamma), _p(ws), ws_bytes, _stream(stream)))


def flint_moe_decode_noalloc(shape, weights, x, batch, out, topk_idx, topk_w, gamma, stream=None):
    """flint_moe_decode on the library's own device scratch (no workspace)."""
    _check("flint_moe_decode_noalloc", lib().flint_moe_decode_noalloc(
        ctypes.byref(shape), ctypes.byref(weights), _p(x), batch, _p(out), _p(topk_idx), _p(topk_w),
        _p(gamma), _stream(stream)))


def flint_moe_decode_stage(stage, shape, weights, x, batch, out, topk_idx, topk_w, gamma, ws,
                           ws_bytes, stream=None):
    _check("flint_moe_decode_stage", lib().flint_moe_decode_stage(
        stage, ctypes.byref(shape), ctypes.byref(weights), _p(x), batch, _p(out), _p(topk_idx),
        _p(topk_w), _p(gamma), _p(ws), ws_bytes, _stream(stream)))


def flint_moe_decode_path(shape: FlintMoeShape, batch: int) -> int:
    v = lib().flint_moe_decode_path(ctypes.byref(shape), int(batch))
    if v < 0:
        raise FlintError("flint_moe_decode_path", -v)
    return v


def flint_moe_decode_stack(shape, layers_dev, n_layers, gammas, x, out, topk_idx, topk_w, layer_out, ws,
                           ws_bytes, stream=None):
    """``layers_dev``: a device uint8 tensor holding ``n_layers``
    FlintMoeWeights structs (see ``weights_table``)."""
    _check("flint_moe_decode_stack",
           lib().flint_moe_decode_stack(ctypes.byref(shape), _p(layers_dev), int(n_layers), _p(gammas), _p(x),
                                        _p(out), _p(topk_idx), _p(topk_w), _p(layer_out), _p(ws),
                                        int(ws_bytes), _stream(stream)))


def weights_table(layers, device) -> torch.Tensor:
    """The FlintMoeWeights structs of ``layers`` (PackedMoeLayer) as a device
    byte tensor, the layout flint_moe_decode_stack reads."""
    arr = (FlintMoeWeights * len(layers))(*[L.weights() for L in layers])
    host = torch.frombuffer(bytearray(bytes(arr)), dtype=torch.uint8)
    return host.to(device)


def flint_moe_prefill(shape, weights, x, n_tokens, out, topk_idx, topk_w, gamma, ws, ws_bytes,
                      stream=None, planes=None):
    """flint_moe_prefill, or flint_moe_prefill_tiled when ``planes`` (a
    FlintPrefillPlanes) is given."""
    if planes is None:
        _check("flint_moe_prefill", lib().flint_moe_prefill(
            ctypes.byref(shape), ctypes.byref(weights), _p(x), n_tokens, _p(out), _p(topk_idx),
            _p(topk_w), _p(gamma), _p(ws), ws_bytes, _stream(stream)))
    else:
        _check("flint_moe_prefill_tiled", lib().flint_moe_prefill_tiled(
            ctypes.byref(shape), ctypes.byref(weights), ctypes.byref(planes), _p(x), n_tokens, _p(out),
            _p(topk_idx), _p(topk_w), _p(gamma), _p(ws), ws_bytes, _stream(stream)))


def flint_moe_prefill_layout(codes, scales, n_mats, rows, cols, interleave, out_codes, out_scales, stream=None):
    _check("flint_moe_prefill_layout", lib().flint_moe_prefill_layout(
        _p(codes), _p(scales), n_mats, rows, cols, interleave, _p(out_codes), _p(out_scales), _stream(stream)))


def flint_dense_gemv(codes, scales, gscale, w_bf16, rows, cols, flags, x, batch, y, epilogue,
                     aux=None, gamma=None, rms_eps=1e-6, stream=None):
    _check("flint_dense_gemv", lib().flint_dense_gemv(
        _p(codes), _p(scales), _p(gscale), _p(w_bf16), rows, cols, flags, _p(x), batch, _p(y),
        epilogue, _p(aux), _p(gamma), ctypes.c_float(rms_eps), _stream(stream)))


def flint_decode_attention_workspace_bytes(shape: FlintAttnShape, window: int, batch: int, max_len: int) -> int:
    n = lib().flint_decode_attention_workspace_bytes(ctypes.byref(shape), window, batch, max_len)
    if n < 0:
        raise FlintError("flint_decode_attention_workspace_bytes", FLINT_ERR_UNSUPPORTED)
    return n


def flint_decode_attention(shape: FlintAttnShape, window, ring, scale, q, batch, k_cache, v_cache, n_rows,
                           seq_base, seq_len, max_len, sinks, out, workspace=None, workspace_bytes=0,
                           error=None, stream=None):
    """Decode attention with learned sinks over a window or the whole
    context (see include/flint_moe.h)."""
    _check("flint_decode_attention", lib().flint_decode_attention(
        ctypes.byref(shape), window, ring, scale, _p(q), batch, _p(k_cache), _p(v_cache), n_rows, _p(seq_base),
        _p(seq_len), max_len, _p(sinks), _p(out), _p(workspace), workspace_bytes, _p(error), _stream(stream)))


def flint_qk_norm_rope_kv(shape: FlintAttnShape, qkv, n_tokens, positions, cos_sin, n_positions, slots,
                          k_cache, v_cache, n_slots, gamma_q, gamma_k, q_out, error=None, stream=None):
    """Per-head Q/K RMSNorm, RoPE (with FLINT_ATTN_ROPE) and the KV-cache
    write of n_tokens projection rows (see include/flint_moe.h)."""
    _check("flint_qk_norm_rope_kv", lib().flint_qk_norm_rope_kv(
        ctypes.byref(shape), _p(qkv), n_tokens, _p(positions), _p(cos_sin), n_positions, _p(slots),
        _p(k_cache), _p(v_cache), n_slots, _p(gamma_q), _p(gamma_k), _p(q_out), _p(error), _stream(stream)))


def flint_stream_read(src, nbytes, threads, loads, blocks, sink, stream=None):
    """A plain read of nbytes of device memory (a measurement utility)."""
    _check("flint_stream_read", lib().flint_stream_read(_p(src), int(nbytes), threads, loads, blocks,
                                                         _p(sink), _stream(stream)))


# ------------------------------------------------------------ conveniences --

def _empty_u8(n: int, device) -> torch.Tensor:
    return torch.empty(int(n), dtype=torch.uint8, device=device)


def repack_matrices(src: torch.Tensor, layout: str = "interleaved", out_codes=None, out_scales=None,
                    mat_stride: int = 1):
    """Repack source super-blocks uint8 [n][rows][cols/64][36] (on the GPU)
    into new (or given) packed planes; returns (codes, scales)."""
    n, rows, nb, _ = src.shape
    cols = nb * 64
    cb, sb = flint_nvfp4_packed_bytes(n, rows, cols)
    if out_codes is None:
        out_codes = _empty_u8(cb, src.device)
        out_scales = _empty_u8(sb, src.device)
    flint_moe_repack(src, n, rows, cols, SRC_LAYOUT_CODES[layout], out_codes, out_scales, mat_stride)
    return out_codes, out_scales


@dataclasses.dataclass
class PackedMoeLayer:
    """Device tensors of one MoE layer in the packed layout (plus, optionally,
    BF16 copies for the W16A16 path) and the matching C structs."""

    hidden: int
    n_experts: int
    inter: int
    shared_inter: int
    router: torch.Tensor
    gu_codes: torch.Tensor
    gu_scales: torch.Tensor
    d_codes: torch.Tensor
    d_scales: torch.Tensor
    gscale: torch.Tensor
    sh_gu_codes: Optional[torch.Tensor] = None
    sh_gu_scales: Optional[torch.Tensor] = None
    sh_d_codes: Optional[torch.Tensor] = None
    sh_d_scales: Optional[torch.Tensor] = None
    sh_gscale: Optional[torch.Tensor] = None
    gu_bf16: Optional[torch.Tensor] = None
    d_bf16: Optional[torch.Tensor] = None
    sh_gu_bf16: Optional[torch.Tensor] = None
    sh_d_bf16: Optional[torch.Tensor] = None

    def shape(self, top_k: int, flags: int = 0, rms_eps: float = 1e-6) -> FlintMoeShape:
        return FlintMoeShape(self.hidden, self.n_experts, self.inter, self.shared_inter, top_k,
                             flags, rms_eps)

    def weights(self) -> FlintMoeWeights:
        w = FlintMoeWeights()
        for f, _ in FlintMoeWeights._fields_:
            t = getattr(self, f)
            setattr(w, f, None if t is None else t.data_ptr())
        return w

    def prefill_planes(self, stream=None):
        """The NVFP4 planes regrouped into the prefill layout (new device
        tensors, flint_moe_prefill_layout).  Returns the FlintPrefillPlanes
        struct and the tensors it points into (keep them alive)."""
        E, H, I, SI = self.n_experts, self.hidden, self.inter, self.shared_inter
        keep = {}
        def one(name, codes, scales, n_mats, rows, cols, interleave):
            oc, os_ = torch.empty_like(codes), torch.empty_like(scales)
            flint_moe_prefill_layout(codes, scales, n_mats, rows, cols, interleave, oc, os_, stream)
            keep[name + "_codes"], keep[name + "_scales"] = oc, os_
        one("gu", self.gu_codes, self.gu_scales, 2 * E, I, H, 1)
        one("d", self.d_codes, self.d_scales, E, H, I, 0)
        if SI > 0:
            one("sh_gu", self.sh_gu_codes, self.sh_gu_scales, 2, SI, H, 1)
            one("sh_d", self.sh_d_codes, self.sh_d_scales, 1, H, SI, 0)
        p = FlintPrefillPlanes()
        for f, _ in FlintPrefillPlanes._fields_:
            t = keep.get(f)
            setattr(p, f, None if t is None else t.data_ptr())
        return p, keep

    def nvfp4_bytes(self) -> int:
        return sum(t.numel() for t in (self.gu_codes, self.gu_scales, self.d_codes, self.d_scales)
                   ) + (0 if self.sh_gu_codes is None else sum(
                       t.numel() for t in (self.sh_gu_codes, self.sh_gu_scales, self.sh_d_codes,
                                           self.sh_d_scales)))

    def add_bf16(self):
        """Attach BF16 copies of the weights (the exact dequantisation of the
        packed NVFP4 matrices, which is exact when the per-tensor scales are
        powers of two) for the W16A16 path."""
        dev = self.gu_codes.device
        H, E, I, SI = self.hidden, self.n_experts, self.inter, self.shared_inter
        gs = self.gscale
        ts_gu = torch.stack([gs[:, 0], gs[:, 1]], 1).reshape(-1).contiguous()
        ts_d = gs[:, 2].contiguous()
        self.gu_bf16 = _dequant_bf16(self.gu_codes, self.gu_scales, 2 * E, I, H, ts_gu, dev)
        self.d_bf16 = _dequant_bf16(self.d_codes, self.d_scales, E, H, I, ts_d, dev)
        if SI:
            sg = self.sh_gscale.reshape(-1)
            self.sh_gu_bf16 = _dequant_bf16(self.sh_gu_codes, self.sh_gu_scales, 2, SI, H,
                                            sg[:2].clone(), dev)
            self.sh_d_bf16 = _dequant_bf16(self.sh_d_codes, self.sh_d_scales, 1, H, SI,
                                           sg[2:3].clone(), dev)
        return self


def _dequant_bf16(codes, scales, n, rows, cols, ts, dev, chunk_mats: int = 16):
    out = torch.empty((n, rows, cols), dtype=torch.bfloat16, device=dev)
    tmp = torch.empty((min(n, chunk_mats), rows, cols), dtype=torch.float32, device=dev)
    cpm, spm = rows * cols // 2, rows * cols // 16
    for m0 in range(0, n, chunk_mats):
        m1 = min(n, m0 + chunk_mats)
        flint_nvfp4_dequant(codes[m0 * cpm:m1 * cpm], scales[m0 * spm:m1 * spm], m1 - m0, rows, cols,
                            ts[m0:m1].clone(), tmp[: m1 - m0])
        out[m0:m1].copy_(tmp[: m1 - m0])
    return out


def pack_moe_layer(router: torch.Tensor, gate: torch.Tensor, up: torch.Tensor, down: torch.Tensor,
                   gscale: torch.Tensor, sh_gate=None, sh_up=None, sh_down=None, sh_gscale=None,
                   layout: str = "interleaved", device="cuda") -> PackedMoeLayer:
    """Upload a layer given in source format (see gen.MoeLayerSource) and
    repack it on the GPU with flint_moe_repack."""
    E, I, nbh, _ = gate.shape
    H = nbh * 64
    SI = 0 if sh_gate is None else sh_gate.shape[1]
    lay = SRC_LAYOUT_CODES[layout]
    dev = torch.device(device)
    gu_c = _empty_u8(2 * E * I * H // 2, dev)
    gu_s = _empty_u8(2 * E * I * H // 16, dev)
    d_c = _empty_u8(E * H * I // 2, dev)
    d_s = _empty_u8(E * H * I // 16, dev)
    g_dev, u_dev, dn_dev = gate.to(dev), up.to(dev), down.to(dev)
    flint_moe_repack(g_dev, E, I, H, lay, gu_c, gu_s, 2)
    flint_moe_repack(u_dev, E, I, H, lay, gu_c[I * H // 2:], gu_s[I * H // 16:], 2)
    flint_moe_repack(dn_dev, E, H, I, lay, d_c, d_s, 1)
    layer = PackedMoeLayer(H, E, I, SI, router.to(dev).contiguous(), gu_c, gu_s, d_c, d_s,
                           gscale.to(dev, torch.float32).contiguous())
    if SI:
        sgc = _empty_u8(2 * SI * H // 2, dev)
        sgs = _empty_u8(2 * SI * H // 16, dev)
        sdc = _empty_u8(H * SI // 2, dev)
        sds = _empty_u8(H * SI // 16, dev)
        flint_moe_repack(sh_gate.to(dev), 1, SI, H, lay, sgc, sgs, 1)
        flint_moe_repack(sh_up.to(dev), 1, SI, H, lay, sgc[SI * H // 2:], sgs[SI * H // 16:], 1)
        flint_moe_repack(sh_down.to(dev), 1, H, SI, lay, sdc, sds, 1)
        sg = torch.zeros(4, dtype=torch.float32, device=dev)   # 16-byte aligned [3] (+pad)
        sg[:3] = sh_gscale.reshape(-1).to(dev, torch.float32)
        layer.sh_gu_codes, layer.sh_gu_scales = sgc, sgs
        layer.sh_d_codes, layer.sh_d_scales = sdc, sds
        layer.sh_gscale = sg
    return layer


def decode_error_word(runner) -> int:
    """The workspace's hand-off error word (1 if a bounded wait ever timed
    out; it stays 0 in normal operation), read through
    flint_moe_workspace_error on the current stream."""
    dst = torch.zeros(1, dtype=torch.int32, device=runner.ws.device)
    flint_moe_workspace_error(runner.ws, runner.ws_bytes, dst)
    return int(dst.item())


class DecodeRunner:
    """Holds a zero-filled workspace and calls flint_moe_decode for a layer."""

    def __init__(self, layer: PackedMoeLayer, top_k: int, flags: int = 0, rms_eps: float = 1e-6):
        self.layer = layer
        self.shape = layer.shape(top_k, flags, rms_eps)
        self.cweights = layer.weights()
        self.ws_bytes = flint_moe_workspace_bytes(self.shape, MAX_DECODE_BATCH)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=layer.router.device)

    def __call__(self, x: torch.Tensor, out: Optional[torch.Tensor] = None, topk_idx=None,
                 topk_w=None, gamma=None, stream=None):
        B = x.shape[0]
        if out is None:
            out = torch.empty_like(x)
        flint_moe_decode(self.shape, self.cweights, x, B, out, topk_idx, topk_w, gamma, self.ws,
                         self.ws_bytes, stream)
        return out

    def stage(self, stage: int, x, out, topk_idx=None, topk_w=None, gamma=None, stream=None):
        flint_moe_decode_stage(stage, self.shape, self.cweights, x, x.shape[0], out, topk_idx,
                               topk_w, gamma, self.ws, self.ws_bytes, stream)


@dataclasses.dataclass
class PackedDenseMlp:
    """A dense SwiGLU MLP in the packed layout: gate/up pair [2][I][H] and
    down [H][I], their FP32 tensor scales, and optional BF16 copies."""

    hidden: int
    inter: int
    gu_codes: torch.Tensor
    gu_scales: torch.Tensor
    d_codes: torch.Tensor
    d_scales: torch.Tensor
    gu_gscale: torch.Tensor      # f32 [4]: gate, up, 0, 0
    d_gscale: torch.Tensor       # f32 [4]: down, 0, 0, 0
    gu_bf16: Optional[torch.Tensor] = None
    d_bf16: Optional[torch.Tensor] = None

    def add_bf16(self):
        dev = self.gu_codes.device
        H, I = self.hidden, self.inter
        self.gu_bf16 = _dequant_bf16(self.gu_codes, self.gu_scales, 2, I, H, self.gu_gscale[:2].clone(), dev)
        self.d_bf16 = _dequant_bf16(self.d_codes, self.d_scales, 1, H, I, self.d_gscale[:1].clone(), dev)
        return self


def pack_dense_mlp(gate: torch.Tensor, up: torch.Tensor, down: torch.Tensor, gscale: torch.Tensor,
                   layout: str = "interleaved", device="cuda") -> PackedDenseMlp:
    """Repack a dense MLP given in source format (gate/up [1][I][H/64][36],
    down [1][H][I/64][36], gscale [1][3]) on the GPU."""
    dev = torch.device(device)
    _, I, nbh, _ = gate.shape
    H = nbh * 64
    gu_c = _empty_u8(2 * I * H // 2, dev)
    gu_s = _empty_u8(2 * I * H // 16, dev)
    repack_matrices(gate.to(dev), layout, gu_c, gu_s)
    repack_matrices(up.to(dev), layout, gu_c[I * H // 2:], gu_s[I * H // 16:])
    d_c, d_s = repack_matrices(down.to(dev), layout)
    g = gscale.reshape(-1).to(dev, torch.float32)
    gg = torch.zeros(4, dtype=torch.float32, device=dev)
    gg[:2] = g[:2]
    gd = torch.zeros(4, dtype=torch.float32, device=dev)
    gd[:1] = g[2:3]
    return PackedDenseMlp(H, I, gu_c, gu_s, d_c, d_s, gg, gd)


class DecodeStep:
    """One decode step over a stack of pre-norm residual sublayers: the MoE
    sublayers, then the dense SwiGLU sublayers (flint_dense_gemv: gate/up
    with the fused RMSNorm, then down with the residual epilogue).  At batch
    1 the MoE sublayers run as one flint_moe_decode_stack launch when the
    shape allows it (``stack``, default: whenever it does); otherwise one
    flint_moe_decode call each (PRE_RMSNORM | RESIDUAL, residual in place).
    Every call enqueues kernels only, so a step can be captured in a graph."""

    def __init__(self, moe_layers, moe_gammas, dense_layers, dense_gammas, top_k: int,
                 flags: int = 0, wbf16: bool = False, rms_eps: float = 1e-6, max_batch: int = 8,
                 stack: Optional[bool] = None):
        self.moe_layers, self.moe_gammas = moe_layers, moe_gammas
        self.dense_layers, self.dense_gammas = dense_layers, dense_gammas
        self.wbf16 = wbf16
        self.eps = rms_eps
        self.top_k = top_k
        f = flags | FLINT_PRE_RMSNORM | FLINT_RESIDUAL | (FLINT_W_BF16 if wbf16 else 0)
        self.shapes = [L.shape(top_k, f, rms_eps) for L in moe_layers]
        self.cweights = [L.weights() for L in moe_layers]
        dev = moe_layers[0].router.device if moe_layers else dense_layers[0].gu_codes.device
        ws = max([flint_moe_workspace_bytes(s, max_batch) for s in self.shapes] + [256])
        self.ws_bytes = ws
        self.ws = torch.zeros(ws, dtype=torch.uint8, device=dev)
        self.h = [torch.empty((max_batch, d.inter), dtype=torch.bfloat16, device=dev)
                  for d in dense_layers]
        K, n = top_k, len(moe_layers)
        self.topk_idx = torch.zeros((n, max_batch * K), dtype=torch.int32, device=dev)
        self.topk_w = torch.zeros((n, max_batch * K), dtype=torch.float32, device=dev)
        self.stack_shape = None
        if moe_layers and not wbf16:
            sshape = moe_layers[0].shape(top_k, flags & FLINT_RENORM, rms_eps)
            ok = flint_moe_decode_path(moe_layers[0].shape(top_k, flags & FLINT_RENORM, rms_eps), 1) \
                == FLINT_PATH_SINGLE_ONE
            if (ok if stack is None else stack) and ok:
                self.stack_shape = sshape
                self.table = weights_table(moe_layers, dev)
                self.gstack = torch.stack([g.reshape(-1) for g in moe_gammas]).contiguous()
                self.stack_idx = torch.zeros((n, K), dtype=torch.int32, device=dev)
                self.stack_w = torch.zeros((n, K), dtype=torch.float32, device=dev)
                self.layer_out = torch.empty((n, moe_layers[0].hidden), dtype=torch.bfloat16, device=dev)
        self.last_stack = False

    def routing(self, layer: int, batch: int):
        """(indices, weights) [batch][K] that MoE sublayer ``layer`` selected
        in the last call."""
        K = self.top_k
        if self.last_stack:
            return self.stack_idx[layer].view(1, K), self.stack_w[layer].view(1, K)
        return (self.topk_idx[layer, :batch * K].view(batch, K), self.topk_w[layer, :batch * K].view(batch, K))

    def __call__(self, x: torch.Tensor, record=None, stream=None):
        """Runs the step on x [B][H] (BF16, updated in place).  If ``record``
        is a list, a copy of the residual entering each sublayer is appended
        (for per-layer checks; not for graph capture)."""
        B = x.shape[0]
        self.last_stack = self.stack_shape is not None and B == 1
        if self.last_stack:
            n = len(self.moe_layers)
            if record is not None:
                record.append(x.clone())
            flint_moe_decode_stack(self.stack_shape, self.table, n, self.gstack, x, x, self.stack_idx,
                                   self.stack_w, self.layer_out if record is not None else None, self.ws,
                                   self.ws_bytes, stream)
            if record is not None:
                for l in range(n - 1):
                    record.append(self.layer_out[l].view(1, -1).clone())
        else:
            for i, (L, g) in enumerate(zip(self.moe_layers, self.moe_gammas)):
                if record is not None:
                    record.append(x.clone())
                flint_moe_decode(self.shapes[i], self.cweights[i], x, B, x, self.topk_idx[i], self.topk_w[i],
                                 g, self.ws, self.ws_bytes, stream)
        fl = FLINT_W_BF16 if self.wbf16 else 0
        for j, (d, g) in enumerate(zip(self.dense_layers, self.dense_gammas)):
            if record is not None:
                record.append(x.clone())
            h = self.h[j][:B]
            flint_dense_gemv(d.gu_codes, d.gu_scales, d.gu_gscale, d.gu_bf16, d.inter, d.hidden,
                             fl | FLINT_PRE_RMSNORM, x, B, h, FLINT_EPI_SWIGLU, gamma=g,
                             rms_eps=self.eps, stream=stream)
            flint_dense_gemv(d.d_codes, d.d_scales, d.d_gscale, d.d_bf16, d.hidden, d.inter, fl, h, B, x,
                             FLINT_EPI_RESIDUAL, aux=x, stream=stream)
        return x


class PrefillRunner:
    """Holds a workspace for up to ``max_tokens`` tokens and calls
    flint_moe_prefill (or, with ``tiled``, flint_moe_prefill_tiled) for a
    layer."""

    def __init__(self, layer: PackedMoeLayer, top_k: int, max_tokens: int, flags: int = 0,
                 rms_eps: float = 1e-6, tiled: bool = False):
        self.layer = layer
        self.shape = layer.shape(top_k, flags, rms_eps)
        self.cweights = layer.weights()
        self.max_tokens = max_tokens
        self.ws_bytes = flint_moe_workspace_bytes(self.shape, max_tokens)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=layer.router.device)
        # tiled: the NVFP4 planes also in the prefill layout (flint_moe_prefill_tiled)
        self.planes, self._planes_keep = layer.prefill_planes() if tiled else (None, None)

    def __call__(self, x: torch.Tensor, out: Optional[torch.Tensor] = None, topk_idx=None, topk_w=None,
                 gamma=None, stream=None):
        T = x.shape[0]
        if T > self.max_tokens:
            raise ValueError(f"{T} tokens > workspace capacity {self.max_tokens}")
        if out is None:
            out = torch.empty_like(x)
        flint_moe_prefill(self.shape, self.cweights, x, T, out, topk_idx, topk_w, gamma, self.ws,
                          self.ws_bytes, stream, planes=self.planes)
        return out
