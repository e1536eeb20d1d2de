"""Thin ctypes binding of libvdn.so (C ABI in include/vdn.h).

The functions here carry the C names and only marshal arguments: torch
tensors become device pointers, the current HIP stream becomes the stream
handle, and a negative status becomes a VdnError.  Every step of the
computation runs in the library's HIP kernels; PyTorch only provides device
memory and streams.  There is no CPU fallback: if the library has not been
built, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # load torch's HIP runtime first so libvdn shares it

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvdn.so")

VDN_F32, VDN_BF16 = 0, 1
VDN_OP_HYBRID, VDN_OP_VDA_SCAN, VDN_OP_WINDOW_ATTN, VDN_OP_DENSE_ATTN, VDN_OP_VDA_BWD = 0, 1, 2, 3, 4
STATUS = {0: "VDN_OK", -1: "VDN_ERR_INVALID_ARG", -2: "VDN_ERR_BAD_SHAPE", -3: "VDN_ERR_DTYPE",
          -4: "VDN_ERR_WORKSPACE", -5: "VDN_ERR_HIP", -6: "VDN_ERR_PARAM_RANGE"}
_TORCH_DTYPE = {VDN_F32: torch.float32, VDN_BF16: torch.bfloat16}


class VdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class vdn_shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("frames", ctypes.c_int32),
        ("tokens_per_frame", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("chunk_frames", ctypes.c_int32), ("window_chunks", ctypes.c_int32),
        ("anchor_first", ctypes.c_int32), ("anchor_last", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("context_tokens", ctypes.c_int32), ("softmax_mxfp8", ctypes.c_int32),
    ]

    @property
    def total_tokens(self) -> int:
        """Rows per (batch, head): video tokens, then context tokens."""
        return self.frames * self.tokens_per_frame + self.context_tokens

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.dtype]


def make_shape(batch, heads, frames, tokens_per_frame, head_dim, dtype="bf16", chunk_frames=5,
               window_chunks=1, anchor_first=True, anchor_last=True, softmax_scale=0.0,
               rms_eps=1e-6, context_tokens=0, softmax_mxfp8=False) -> vdn_shape:
    dt = {"f32": VDN_F32, "bf16": VDN_BF16, torch.float32: VDN_F32, torch.bfloat16: VDN_BF16}.get(dtype, dtype)
    return vdn_shape(batch, heads, frames, tokens_per_frame, head_dim, chunk_frames, window_chunks,
                     int(anchor_first), int(anchor_last), softmax_scale, rms_eps, dt, context_tokens,
                     int(bool(softmax_mxfp8)))


def shape_from_config(cfg, softmax_mxfp8=False) -> vdn_shape:
    """vdn_shape of a synth.VdnConfig."""
    return make_shape(cfg.batch, cfg.heads, cfg.frames, cfg.tokens_per_frame, cfg.head_dim,
                      cfg.dtype, cfg.chunk_frames, cfg.window_chunks, cfg.anchor_first,
                      cfg.anchor_last, 0.0, cfg.rms_eps, cfg.context_tokens, softmax_mxfp8)


class vdn_phase_stat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_float)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m video_diffusion_hybrid_vda_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    P, S, I, SZ = ctypes.c_void_p, ctypes.POINTER(vdn_shape), ctypes.c_int, ctypes.c_size_t
    lib.vdn_workspace_bytes.argtypes = [S, I]
    lib.vdn_workspace_bytes.restype = SZ
    lib.vdn_hybrid_attn_fwd.argtypes = [S] + [P] * 12 + [P, SZ, P]
    lib.vdn_hybrid_attn_fwd.restype = I
    lib.vda_scan_fwd.argtypes = [S] + [P] * 9 + [P, SZ, P]
    lib.vda_scan_fwd.restype = I
    lib.vda_scan_fwd_noalloc.argtypes = [S] + [P] * 9 + [P]
    lib.vda_scan_fwd_noalloc.restype = I
    lib.vda_scan_bwd.argtypes = [S] + [P] * 13 + [P, SZ, P]
    lib.vda_scan_bwd.restype = I
    lib.window_anchor_attn_fwd.argtypes = [S] + [P] * 6 + [P, SZ, P]
    lib.window_anchor_attn_fwd.restype = I
    lib.vdn_mxfp8_quantize.argtypes = [P, ctypes.c_int64, P, P, P]
    lib.vdn_mxfp8_quantize.restype = I
    lib.window_anchor_attn_mxfp8_fwd.argtypes = [S] + [P] * 8 + [P, SZ, P]
    lib.window_anchor_attn_mxfp8_fwd.restype = I
    lib.vdn_dense_attn_fwd.argtypes = [S] + [P] * 6 + [SZ, P]
    lib.vdn_dense_attn_fwd.restype = I
    lib.vdn_set_param_check.argtypes = [I]
    lib.vdn_set_param_check.restype = I
    lib.vdn_last_error.argtypes = []
    lib.vdn_last_error.restype = ctypes.c_char_p
    lib.vdn_version.argtypes = []
    lib.vdn_version.restype = ctypes.c_char_p
    lib.vdn_timing_start.argtypes = []
    lib.vdn_timing_start.restype = I
    lib.vdn_timing_stop.argtypes = [ctypes.POINTER(vdn_phase_stat), I]
    lib.vdn_timing_stop.restype = I
    return lib


_lib = _load()

EXPORTS = ("vdn_workspace_bytes", "vdn_hybrid_attn_fwd", "vda_scan_fwd", "window_anchor_attn_fwd",
           "vdn_dense_attn_fwd", "vdn_set_param_check", "vdn_last_error", "vdn_version",
           "vdn_timing_start", "vdn_timing_stop", "vdn_mxfp8_quantize", "window_anchor_attn_mxfp8_fwd",
           "vda_scan_bwd", "vda_scan_fwd_noalloc")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != 0:
        raise VdnError(status, vdn_last_error())
    return status


def vdn_last_error() -> str:
    return _lib.vdn_last_error().decode()


def vdn_version() -> str:
    return _lib.vdn_version().decode()


def vdn_timing_start() -> int:
    return _check(_lib.vdn_timing_start())


def vdn_timing_stop() -> dict:
    """{phase name: (launches, total ms)} of the phases recorded since start."""
    stats = (vdn_phase_stat * 32)()
    n = _lib.vdn_timing_stop(stats, 32)
    if n < 0:
        raise VdnError(n, vdn_last_error())
    return {stats[i].name.decode(): (stats[i].launches, stats[i].total_ms) for i in range(n)}


def vdn_workspace_bytes(shape: vdn_shape, op: int) -> int:
    n = _lib.vdn_workspace_bytes(ctypes.byref(shape), op)
    if n == 0:
        raise VdnError(-2, vdn_last_error())
    return n


def workspace(shape: vdn_shape, op: int, device="cuda") -> torch.Tensor:
    """Allocate (through torch) a device workspace of the size the library asks for."""
    return torch.empty(vdn_workspace_bytes(shape, op), dtype=torch.uint8, device=device)


def vdn_hybrid_attn_fwd(shape, x, q, k, v, gamma, beta, w_gs, w_gl, rms_w, w_os, w_ol, out, ws,
                        stream=None) -> int:
    return _check(_lib.vdn_hybrid_attn_fwd(
        ctypes.byref(shape), _ptr(x), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta),
        _ptr(w_gs), _ptr(w_gl), _ptr(rms_w), _ptr(w_os), _ptr(w_ol), _ptr(out),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def vda_scan_fwd(shape, q, k, v, gamma, beta, rms_w, gate_l, out, states, ws, stream=None) -> int:
    return _check(_lib.vda_scan_fwd(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta), _ptr(rms_w),
        _ptr(gate_l), _ptr(out), _ptr(states), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def vda_scan_fwd_noalloc(shape, q, k, v, gamma, beta, rms_w, gate_l, out, states, stream=None) -> int:
    return _check(_lib.vda_scan_fwd_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta), _ptr(rms_w),
        _ptr(gate_l), _ptr(out), _ptr(states), _stream(stream)))


def vda_scan_bwd(shape, q, k, v, gamma, beta, rms_w, d_out, dq, dk, dv, dgamma, dbeta, drms_w, ws,
                 stream=None) -> int:
    return _check(_lib.vda_scan_bwd(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta), _ptr(rms_w),
        _ptr(d_out), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgamma), _ptr(dbeta), _ptr(drms_w), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def window_anchor_attn_fwd(shape, q, k, v, gate_s, out, lse, ws, stream=None) -> int:
    return _check(_lib.window_anchor_attn_fwd(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(gate_s), _ptr(out), _ptr(lse),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def vdn_mxfp8_quantize(x, n_elems, codes, scales, stream=None) -> int:
    return _check(_lib.vdn_mxfp8_quantize(_ptr(x), int(n_elems), _ptr(codes), _ptr(scales), _stream(stream)))


def window_anchor_attn_mxfp8_fwd(shape, q_codes, q_scales, k_codes, k_scales, v, gate_s, out, lse, ws,
                                 stream=None) -> int:
    return _check(_lib.window_anchor_attn_mxfp8_fwd(
        ctypes.byref(shape), _ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales), _ptr(v),
        _ptr(gate_s), _ptr(out), _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def vdn_dense_attn_fwd(shape, q, k, v, w_o, out, ws, stream=None) -> int:
    return _check(_lib.vdn_dense_attn_fwd(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(w_o), _ptr(out), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def vdn_set_param_check(on: bool) -> bool:
    """Turn the device-side gamma/beta range check on or off; returns the previous setting."""
    return bool(_lib.vdn_set_param_check(int(bool(on))))


# ---- convenience wrappers: allocate outputs and workspace through torch, then call

def hybrid_attn(shape, inp: dict, ws=None, stream=None) -> torch.Tensor:
    B, L = shape.batch, shape.total_tokens
    D = shape.heads * shape.head_dim
    out = torch.empty(B, L, D, dtype=shape.torch_dtype, device=inp["q"].device)
    ws = workspace(shape, VDN_OP_HYBRID, inp["q"].device) if ws is None else ws
    vdn_hybrid_attn_fwd(shape, inp["x"], inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"],
                        inp["w_gs"], inp["w_gl"], inp.get("rms_w"), inp["w_os"], inp["w_ol"], out,
                        ws, stream)
    return out


def vda_scan(shape, inp: dict, gate_l=None, with_states=False, ws=None, stream=None):
    B, H, T, d = shape.batch, shape.heads, shape.frames, shape.head_dim
    L = shape.total_tokens
    dev = inp["q"].device
    out = torch.empty(B, L, H * d, dtype=shape.torch_dtype, device=dev)
    states = torch.empty(2, B, H, T, d, d, dtype=torch.float32, device=dev) if with_states else None
    ws = workspace(shape, VDN_OP_VDA_SCAN, dev) if ws is None else ws
    vda_scan_fwd(shape, inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], inp.get("rms_w"),
                 gate_l, out, states, ws, stream)
    return (out, states) if with_states else out


def vda_scan_grad(shape, inp: dict, d_out, ws=None, stream=None) -> dict:
    """Gradient of <d_out, ungated linear-branch output> with respect to q, k, v, gamma, beta and
    the RMSNorm weight (d_out [B, Lt, D] like the forward output)."""
    B, H, T, d = shape.batch, shape.heads, shape.frames, shape.head_dim
    dev = inp["q"].device
    g = {n: torch.empty_like(inp[n]) for n in ("q", "k", "v")}
    g["gamma"] = torch.empty(B, H, T, dtype=torch.float32, device=dev)
    g["beta"] = torch.empty(B, H, T, dtype=torch.float32, device=dev)
    g["rms_w"] = torch.empty(H * d, dtype=torch.float32, device=dev)
    ws = workspace(shape, VDN_OP_VDA_BWD, dev) if ws is None else ws
    vda_scan_bwd(shape, inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], inp.get("rms_w"), d_out,
                 g["q"], g["k"], g["v"], g["gamma"], g["beta"], g["rms_w"], ws, stream)
    return g


def window_attn(shape, inp: dict, gate_s=None, with_lse=False, ws=None, stream=None):
    B, H, d = shape.batch, shape.heads, shape.head_dim
    L = shape.total_tokens
    dev = inp["q"].device
    out = torch.empty(B, L, H * d, dtype=shape.torch_dtype, device=dev)
    lse = torch.empty(B, H, L, dtype=torch.float32, device=dev) if with_lse else None
    ws = workspace(shape, VDN_OP_WINDOW_ATTN, dev) if ws is None else ws
    window_anchor_attn_fwd(shape, inp["q"], inp["k"], inp["v"], gate_s, out, lse, ws, stream)
    return (out, lse) if with_lse else out


def dense_attn(shape, inp: dict, w_o, ws=None, stream=None) -> torch.Tensor:
    B, L = shape.batch, shape.total_tokens
    D = shape.heads * shape.head_dim
    dev = inp["q"].device
    out = torch.empty(B, L, D, dtype=shape.torch_dtype, device=dev)
    ws = workspace(shape, VDN_OP_DENSE_ATTN, dev) if ws is None else ws
    vdn_dense_attn_fwd(shape, inp["q"], inp["k"], inp["v"], w_o, out, ws, stream)
    return out


def mxfp8_quantize(x: torch.Tensor, stream=None):
    """MXFP8 of a bf16 tensor along its last axis (a multiple of 32):
    (codes uint8 of x's shape, scales uint8 [..., last / 32])."""
    assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.shape[-1] % 32 == 0
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1] + (x.shape[-1] // 32,), dtype=torch.uint8, device=x.device)
    vdn_mxfp8_quantize(x, x.numel(), codes, scales, stream)
    return codes, scales


def window_attn_mxfp8(shape, q_codes, q_scales, k_codes, k_scales, v, gate_s=None, with_lse=False,
                      ws=None, stream=None):
    B, H, d = shape.batch, shape.heads, shape.head_dim
    L = shape.total_tokens
    dev = v.device
    out = torch.empty(B, L, H * d, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, H, L, dtype=torch.float32, device=dev) if with_lse else None
    if ws is None:
        plain = vdn_shape.from_buffer_copy(shape)
        plain.softmax_mxfp8 = 0
        ws = workspace(plain, VDN_OP_WINDOW_ATTN, dev)
    window_anchor_attn_mxfp8_fwd(shape, q_codes, q_scales, k_codes, k_scales, v, gate_s, out, lse, ws, stream)
    return (out, lse) if with_lse else out
