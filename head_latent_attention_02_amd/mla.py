"""Thin ctypes binding of libmla (include/mla.h).

Argument marshalling only: every step of the MLA forward runs in the HIP
kernels of libmla.so.  PyTorch supplies device memory and the current stream.
If the library is missing the first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla.so")

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE_TOO_SMALL = 3
MLA_ERR_HIP = 4

MLA_BF16 = 0
MLA_FP32 = 1

# bytes of the library's fixed decode scratch (MLA_DECODE_NOALLOC_MAX_BYTES)
DECODE_NOALLOC_MAX_BYTES = 64 << 20

MLA_ALGO_AUTO = 0
MLA_ALGO_SIMT = 1
MLA_ALGO_MFMA = 2
MLA_ALGO_FUSED = 3     # explicit forward with the up-projection inside the attention kernel

EXPORTED_SYMBOLS = (
    "mla_fwd_explicit_workspace_size", "mla_fwd_explicit", "mla_fwd_explicit_workspace_layout",
    "mla_decode_absorbed_workspace_size", "mla_decode_absorbed", "mla_decode_absorbed_workspace_layout",
    "mla_fwd_absorbed_workspace_size", "mla_fwd_absorbed", "mla_decode_absorbed_noalloc",
    "mla_bwd_explicit_workspace_size", "mla_bwd_explicit",
    "mla_status_string", "mla_last_error", "mla_build_info",
    "mla_timing_begin", "mla_timing_end", "mla_timing_reset", "mla_timing_count", "mla_timing_get",
)


class MlaExplicitDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("s_q", ctypes.c_int32), ("s_kv", ctypes.c_int32),
        ("n_heads", ctypes.c_int32), ("d_kv", ctypes.c_int32), ("d_nope", ctypes.c_int32),
        ("d_rope", ctypes.c_int32), ("d_v", ctypes.c_int32), ("q_pos0", ctypes.c_int64),
        ("kv_pos0", ctypes.c_int64), ("causal", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("rope_base", ctypes.c_float), ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
        ("algo", ctypes.c_int),
    ]


class MlaDecodeDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("d_kv", ctypes.c_int32),
        ("d_nope", ctypes.c_int32), ("d_rope", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("max_cache_len", ctypes.c_int32), ("cache_batch_stride", ctypes.c_int64),
        ("n_splits", ctypes.c_int32), ("softmax_scale", ctypes.c_float), ("rope_base", ctypes.c_float),
        ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int), ("algo", ctypes.c_int),
    ]


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _lib()
        msg = lib.mla_status_string(status).decode()
        detail = lib.mla_last_error().decode()
        super().__init__(f"{where}: {msg}" + (f" ({detail})" if detail else ""))
        self.status = status


_LIB: Optional[ctypes.CDLL] = None


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmla.so not built at {LIB_PATH}; run `python -m head_latent_attention_02_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        lib.mla_fwd_explicit_workspace_size.argtypes = [ctypes.POINTER(MlaExplicitDesc)]
        lib.mla_fwd_explicit_workspace_size.restype = sz
        lib.mla_fwd_explicit.argtypes = [ctypes.POINTER(MlaExplicitDesc), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.mla_fwd_explicit.restype = ctypes.c_int
        lib.mla_fwd_absorbed_workspace_size.argtypes = [ctypes.POINTER(MlaExplicitDesc)]
        lib.mla_fwd_absorbed_workspace_size.restype = sz
        lib.mla_fwd_absorbed.argtypes = [ctypes.POINTER(MlaExplicitDesc), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.mla_fwd_absorbed.restype = ctypes.c_int
        lib.mla_bwd_explicit_workspace_size.argtypes = [ctypes.POINTER(MlaExplicitDesc)]
        lib.mla_bwd_explicit_workspace_size.restype = sz
        lib.mla_bwd_explicit.argtypes = [ctypes.POINTER(MlaExplicitDesc)] + [vp] * 14 + [sz, vp]
        lib.mla_bwd_explicit.restype = ctypes.c_int
        lib.mla_fwd_explicit_workspace_layout.argtypes = [ctypes.POINTER(MlaExplicitDesc), ctypes.POINTER(sz)]
        lib.mla_fwd_explicit_workspace_layout.restype = ctypes.c_int
        lib.mla_decode_absorbed_workspace_size.argtypes = [ctypes.POINTER(MlaDecodeDesc)]
        lib.mla_decode_absorbed_workspace_size.restype = sz
        lib.mla_decode_absorbed.argtypes = [ctypes.POINTER(MlaDecodeDesc), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.mla_decode_absorbed.restype = ctypes.c_int
        lib.mla_decode_absorbed_noalloc.argtypes = [ctypes.POINTER(MlaDecodeDesc), vp, vp, vp, vp, vp, vp, vp, vp]
        lib.mla_decode_absorbed_noalloc.restype = ctypes.c_int
        lib.mla_decode_absorbed_workspace_layout.argtypes = [ctypes.POINTER(MlaDecodeDesc), ctypes.POINTER(sz)]
        lib.mla_decode_absorbed_workspace_layout.restype = ctypes.c_int
        lib.mla_status_string.argtypes = [ctypes.c_int]
        lib.mla_status_string.restype = ctypes.c_char_p
        lib.mla_last_error.argtypes = []
        lib.mla_last_error.restype = ctypes.c_char_p
        lib.mla_build_info.argtypes = []
        lib.mla_build_info.restype = ctypes.c_char_p
        for f in ("mla_timing_begin", "mla_timing_end", "mla_timing_reset"):
            getattr(lib, f).argtypes = []
            getattr(lib, f).restype = ctypes.c_int
        lib.mla_timing_count.argtypes = []
        lib.mla_timing_count.restype = ctypes.c_int32
        lib.mla_timing_get.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_char_p),
                                       ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        lib.mla_timing_get.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def library() -> ctypes.CDLL:
    """The loaded libmla handle (loads it on first use)."""
    return _lib()


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return MLA_BF16
    if t == torch.float32:
        return MLA_FP32
    raise TypeError(f"unsupported dtype {t}")


def _torch_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == MLA_BF16 else torch.float32


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(status: int, where: str):
    if status != MLA_OK:
        raise MlaError(status, where)


def _expect(t, name: str, shape: tuple, dtype: torch.dtype, device: torch.device):
    """Raise ValueError unless ``t`` is a dense row-major tensor of exactly
    ``shape`` and ``dtype`` on ``device``: the library reads and writes these
    buffers through raw pointers with the sizes the descriptor states."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _expect_workspace(ws, device: torch.device):
    if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.dim() != 1:
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor (its length is its size in bytes)")
    if ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, expected {device}")


def _expect_cuda(device: torch.device):
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {device}")


# ----------------------------------------------------------------- explicit --
def explicit_desc(*, batch, s_q, s_kv, n_heads, d_kv, d_nope, d_rope, d_v, q_pos0=0, kv_pos0=0,
                  causal=True, softmax_scale=None, rope_base=10000.0, in_dtype=MLA_BF16,
                  out_dtype=MLA_FP32, algo=MLA_ALGO_AUTO) -> MlaExplicitDesc:
    if softmax_scale is None:
        softmax_scale = (d_nope + d_rope) ** -0.5
    return MlaExplicitDesc(batch, s_q, s_kv, n_heads, d_kv, d_nope, d_rope, d_v, q_pos0, kv_pos0,
                           int(causal), softmax_scale, rope_base, in_dtype, out_dtype, algo)


def mla_fwd_explicit_workspace_size(desc: MlaExplicitDesc) -> int:
    return int(_lib().mla_fwd_explicit_workspace_size(ctypes.byref(desc)))


def mla_fwd_explicit_workspace_layout(desc: MlaExplicitDesc) -> tuple:
    off = (ctypes.c_size_t * 4)()
    _check(_lib().mla_fwd_explicit_workspace_layout(ctypes.byref(desc), off), "mla_fwd_explicit_workspace_layout")
    return tuple(int(x) for x in off)


def mla_fwd_absorbed_workspace_size(desc: MlaExplicitDesc) -> int:
    return int(_lib().mla_fwd_absorbed_workspace_size(ctypes.byref(desc)))


def mla_fwd_absorbed(q_nope: torch.Tensor, q_pe: torch.Tensor, c_kv: torch.Tensor, k_pe: torch.Tensor,
                     w_kv_b: torch.Tensor, **kw):
    """Absorbed-form forward of the explicit problem; see mla_fwd_absorbed in
    include/mla.h.  Same arguments and results as mla_fwd_explicit."""
    return _fwd(False, q_nope, q_pe, c_kv, k_pe, w_kv_b, **kw)


def mla_fwd_explicit(q_nope: torch.Tensor, q_pe: torch.Tensor, c_kv: torch.Tensor, k_pe: torch.Tensor,
                     w_kv_b: torch.Tensor, **kw):
    """Explicit-form MLA forward; see mla_fwd_explicit in include/mla.h.

    Shapes: q_nope [B,S_q,H,d_nope], q_pe [B,S_q,H,d_rope], c_kv [B,S_kv,d_kv],
    k_pe [B,S_kv,d_rope], w_kv_b [H*(d_nope+d_v), d_kv].  Keywords: q_pos0,
    kv_pos0, causal, softmax_scale, rope_base, out_dtype, algo, return_lse,
    out, lse, workspace.  Returns (out, lse, workspace); lse is None when
    return_lse is False.
    """
    return _fwd(True, q_nope, q_pe, c_kv, k_pe, w_kv_b, **kw)


def _fwd(explicit: bool, q_nope: torch.Tensor, q_pe: torch.Tensor, c_kv: torch.Tensor, k_pe: torch.Tensor,
         w_kv_b: torch.Tensor, *, q_pos0: int = 0, kv_pos0: int = 0, causal: bool = True,
         softmax_scale: Optional[float] = None, rope_base: float = 10000.0,
         out_dtype: torch.dtype = torch.float32, algo: int = MLA_ALGO_AUTO,
         return_lse: bool = True, out: Optional[torch.Tensor] = None,
         lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    if q_nope.dim() != 4 or q_pe.dim() != 4 or c_kv.dim() != 3 or k_pe.dim() != 3 or w_kv_b.dim() != 2:
        raise ValueError("expected q_nope, q_pe [B,S_q,H,*], c_kv, k_pe [B,S_kv,*], w_kv_b [H*(d_nope+d_v), d_kv]")
    B, S_q, H, d_nope = q_nope.shape
    S_kv, d_kv = c_kv.shape[1], c_kv.shape[2]
    d_rope = q_pe.shape[-1]
    if H < 1 or w_kv_b.shape[0] % H != 0 or w_kv_b.shape[0] // H <= d_nope:
        raise ValueError(f"w_kv_b rows ({w_kv_b.shape[0]}) must be H*(d_nope+d_v) with H={H}, d_nope={d_nope}")
    d_v = w_kv_b.shape[0] // H - d_nope
    dt = _dtype_code(q_nope.dtype)
    dev = q_nope.device
    _expect(q_nope, "q_nope", (B, S_q, H, d_nope), q_nope.dtype, dev)
    _expect(q_pe, "q_pe", (B, S_q, H, d_rope), q_nope.dtype, dev)
    _expect(c_kv, "c_kv", (B, S_kv, d_kv), q_nope.dtype, dev)
    _expect(k_pe, "k_pe", (B, S_kv, d_rope), q_nope.dtype, dev)
    _expect(w_kv_b, "w_kv_b", (H * (d_nope + d_v), d_kv), q_nope.dtype, dev)
    if out is not None:
        _expect(out, "out", (B, S_q, H, d_v), out_dtype, dev)
    if return_lse and lse is not None:
        _expect(lse, "lse", (B, H, S_q), torch.float32, dev)
    if workspace is not None:
        _expect_workspace(workspace, dev)
    _expect_cuda(dev)
    desc = explicit_desc(batch=B, s_q=S_q, s_kv=S_kv, n_heads=H, d_kv=d_kv, d_nope=d_nope, d_rope=d_rope,
                         d_v=d_v, q_pos0=q_pos0, kv_pos0=kv_pos0, causal=causal, softmax_scale=softmax_scale,
                         rope_base=rope_base, in_dtype=dt, out_dtype=_dtype_code(out_dtype), algo=algo)
    name = "mla_fwd_explicit" if explicit else "mla_fwd_absorbed"
    ws_bytes = (mla_fwd_explicit_workspace_size if explicit else mla_fwd_absorbed_workspace_size)(desc)
    if ws_bytes == 0 and S_q > 0:
        _check(MLA_ERR_INVALID_ARGUMENT if algo not in (MLA_ALGO_MFMA, MLA_ALGO_FUSED) else MLA_ERR_UNSUPPORTED,
               name + "_workspace_size")
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((B, S_q, H, d_v), dtype=out_dtype, device=dev)
    if return_lse and lse is None:
        lse = torch.empty((B, H, S_q), dtype=torch.float32, device=dev)
    st = getattr(_lib(), name)(ctypes.byref(desc), _ptr(q_nope), _ptr(q_pe), _ptr(c_kv), _ptr(k_pe),
                               _ptr(w_kv_b), _ptr(out), _ptr(lse) if return_lse else None,
                               workspace.data_ptr(), workspace.numel(), _stream(dev))
    _check(st, name)
    return out, (lse if return_lse else None), workspace


def mla_bwd_explicit_workspace_size(desc: MlaExplicitDesc) -> int:
    return int(_lib().mla_bwd_explicit_workspace_size(ctypes.byref(desc)))


def mla_bwd_explicit(q_nope: torch.Tensor, q_pe: torch.Tensor, c_kv: torch.Tensor, k_pe: torch.Tensor,
                     w_kv_b: torch.Tensor, out: torch.Tensor, lse: torch.Tensor, d_out: torch.Tensor, *,
                     q_pos0: int = 0, kv_pos0: int = 0, causal: bool = True,
                     softmax_scale: Optional[float] = None, rope_base: float = 10000.0,
                     algo: int = MLA_ALGO_AUTO, grads: Optional[dict] = None,
                     workspace: Optional[torch.Tensor] = None):
    """Explicit-form backward; see mla_bwd_explicit in include/mla.h.

    Inputs as for mla_fwd_explicit plus the forward's out [B,S_q,H,d_v] and
    lse [B,H,S_q] (fp32) and d_out (out's dtype).  Returns (grads, workspace)
    with grads a dict of fp32 tensors dq_nope, dq_pe, dc_kv, dk_pe, dw_kv_b
    (caller-supplied ones in `grads` are checked and written in place).
    """
    if q_nope.dim() != 4 or q_pe.dim() != 4 or c_kv.dim() != 3 or k_pe.dim() != 3 or w_kv_b.dim() != 2:
        raise ValueError("expected q_nope, q_pe [B,S_q,H,*], c_kv, k_pe [B,S_kv,*], w_kv_b [H*(d_nope+d_v), d_kv]")
    B, S_q, H, d_nope = q_nope.shape
    S_kv, d_kv = c_kv.shape[1], c_kv.shape[2]
    d_rope = q_pe.shape[-1]
    if H < 1 or w_kv_b.shape[0] % H != 0 or w_kv_b.shape[0] // H <= d_nope:
        raise ValueError(f"w_kv_b rows ({w_kv_b.shape[0]}) must be H*(d_nope+d_v) with H={H}, d_nope={d_nope}")
    d_v = w_kv_b.shape[0] // H - d_nope
    dev = q_nope.device
    _expect(q_nope, "q_nope", (B, S_q, H, d_nope), q_nope.dtype, dev)
    _expect(q_pe, "q_pe", (B, S_q, H, d_rope), q_nope.dtype, dev)
    _expect(c_kv, "c_kv", (B, S_kv, d_kv), q_nope.dtype, dev)
    _expect(k_pe, "k_pe", (B, S_kv, d_rope), q_nope.dtype, dev)
    _expect(w_kv_b, "w_kv_b", (H * (d_nope + d_v), d_kv), q_nope.dtype, dev)
    _expect(out, "out", (B, S_q, H, d_v), out.dtype, dev)
    _expect(d_out, "d_out", (B, S_q, H, d_v), out.dtype, dev)
    _expect(lse, "lse", (B, H, S_q), torch.float32, dev)
    shapes = {"dq_nope": (B, S_q, H, d_nope), "dq_pe": (B, S_q, H, d_rope), "dc_kv": (B, S_kv, d_kv),
              "dk_pe": (B, S_kv, d_rope), "dw_kv_b": (H * (d_nope + d_v), d_kv)}
    grads = dict(grads or {})
    for k, shp in shapes.items():
        if k in grads:
            _expect(grads[k], k, shp, torch.float32, dev)
    if workspace is not None:
        _expect_workspace(workspace, dev)
    _expect_cuda(dev)
    desc = explicit_desc(batch=B, s_q=S_q, s_kv=S_kv, n_heads=H, d_kv=d_kv, d_nope=d_nope, d_rope=d_rope,
                         d_v=d_v, q_pos0=q_pos0, kv_pos0=kv_pos0, causal=causal, softmax_scale=softmax_scale,
                         rope_base=rope_base, in_dtype=_dtype_code(q_nope.dtype), out_dtype=_dtype_code(out.dtype),
                         algo=algo)
    ws_bytes = mla_bwd_explicit_workspace_size(desc)
    if ws_bytes == 0:
        _check(MLA_ERR_INVALID_ARGUMENT if algo not in (MLA_ALGO_MFMA, MLA_ALGO_FUSED) else MLA_ERR_UNSUPPORTED,
               "mla_bwd_explicit_workspace_size")
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    for k, shp in shapes.items():
        if k not in grads:
            grads[k] = torch.empty(shp, dtype=torch.float32, device=dev)
    st = _lib().mla_bwd_explicit(ctypes.byref(desc), _ptr(q_nope), _ptr(q_pe), _ptr(c_kv), _ptr(k_pe),
                                 _ptr(w_kv_b), _ptr(out), _ptr(lse), _ptr(d_out), _ptr(grads["dq_nope"]),
                                 _ptr(grads["dq_pe"]), _ptr(grads["dc_kv"]), _ptr(grads["dk_pe"]),
                                 _ptr(grads["dw_kv_b"]), workspace.data_ptr(), workspace.numel(), _stream(dev))
    _check(st, "mla_bwd_explicit")
    return grads, workspace


# ------------------------------------------------------------------- decode --
def decode_desc(*, batch, n_heads, d_kv, d_nope, d_rope, d_v, max_cache_len, cache_batch_stride=None,
                n_splits=16, softmax_scale=None, rope_base=10000.0, in_dtype=MLA_BF16, out_dtype=MLA_FP32,
                algo=MLA_ALGO_AUTO) -> MlaDecodeDesc:
    if softmax_scale is None:
        softmax_scale = (d_nope + d_rope) ** -0.5
    if cache_batch_stride is None:
        cache_batch_stride = max_cache_len * (d_kv + d_rope)
    return MlaDecodeDesc(batch, n_heads, d_kv, d_nope, d_rope, d_v, max_cache_len, cache_batch_stride,
                         n_splits, softmax_scale, rope_base, in_dtype, out_dtype, algo)


def mla_decode_absorbed_workspace_size(desc: MlaDecodeDesc) -> int:
    return int(_lib().mla_decode_absorbed_workspace_size(ctypes.byref(desc)))


def mla_decode_absorbed_workspace_layout(desc: MlaDecodeDesc) -> tuple:
    off = (ctypes.c_size_t * 4)()
    _check(_lib().mla_decode_absorbed_workspace_layout(ctypes.byref(desc), off),
           "mla_decode_absorbed_workspace_layout")
    return tuple(int(x) for x in off)


def mla_decode_absorbed(q_nope: torch.Tensor, q_pe: torch.Tensor, kv_cache: torch.Tensor,
                        cache_len: torch.Tensor, w_kv_b: torch.Tensor, *, n_splits: int = 16,
                        d_kv: Optional[int] = None, softmax_scale: Optional[float] = None,
                        rope_base: float = 10000.0, out_dtype: torch.dtype = torch.float32,
                        algo: int = MLA_ALGO_AUTO, return_lse: bool = True,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None):
    """Absorbed split-KV decode step; see mla_decode_absorbed in include/mla.h.

    q_nope [B,H,d_nope], q_pe [B,H,d_rope], kv_cache [B,L_max,d_kv+d_rope] (its
    sequence stride may exceed L_max rows; rows must be contiguous),
    cache_len [B] int32 on the device, w_kv_b [H*(d_nope+d_v), d_kv].
    """
    desc, d_v = _decode_checked_desc(q_nope, q_pe, kv_cache, cache_len, w_kv_b, n_splits=n_splits, d_kv=d_kv,
                                     softmax_scale=softmax_scale, rope_base=rope_base, out_dtype=out_dtype,
                                     algo=algo, return_lse=return_lse, out=out, lse=lse, workspace=workspace)
    B, H = q_nope.shape[0], q_nope.shape[1]
    dev = q_nope.device
    ws_bytes = mla_decode_absorbed_workspace_size(desc)
    if ws_bytes == 0:
        _check(MLA_ERR_INVALID_ARGUMENT if algo not in (MLA_ALGO_MFMA, MLA_ALGO_FUSED) else MLA_ERR_UNSUPPORTED,
               "mla_decode_absorbed_workspace_size")
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((B, H, d_v), dtype=out_dtype, device=dev)
    if return_lse and lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    st = _lib().mla_decode_absorbed(ctypes.byref(desc), _ptr(q_nope), _ptr(q_pe), _ptr(kv_cache),
                                    _ptr(cache_len), _ptr(w_kv_b), _ptr(out), _ptr(lse) if return_lse else None,
                                    workspace.data_ptr(), workspace.numel(), _stream(dev))
    _check(st, "mla_decode_absorbed")
    return out, (lse if return_lse else None), workspace


def mla_decode_absorbed_noalloc(q_nope: torch.Tensor, q_pe: torch.Tensor, kv_cache: torch.Tensor,
                                cache_len: torch.Tensor, w_kv_b: torch.Tensor, out: torch.Tensor,
                                lse: Optional[torch.Tensor] = None, *, n_splits: int = 16,
                                d_kv: Optional[int] = None, softmax_scale: Optional[float] = None,
                                rope_base: float = 10000.0, algo: int = MLA_ALGO_AUTO) -> None:
    """The decode step without a workspace, for callers that cannot allocate;
    see mla_decode_absorbed_noalloc in include/mla.h.  The caller passes the
    outputs (out [B,H,d_v], lse [B,H] fp32 or None); nothing is allocated here
    or in the library.  Calls on one GPU share the library's fixed scratch and
    must not overlap."""
    if out is None:
        raise ValueError("out must be given: this entry point allocates nothing")
    desc, _ = _decode_checked_desc(q_nope, q_pe, kv_cache, cache_len, w_kv_b, n_splits=n_splits, d_kv=d_kv,
                                   softmax_scale=softmax_scale, rope_base=rope_base, out_dtype=out.dtype,
                                   algo=algo, return_lse=lse is not None, out=out, lse=lse, workspace=None)
    st = _lib().mla_decode_absorbed_noalloc(ctypes.byref(desc), _ptr(q_nope), _ptr(q_pe), _ptr(kv_cache),
                                            _ptr(cache_len), _ptr(w_kv_b), _ptr(out), _ptr(lse),
                                            _stream(q_nope.device))
    _check(st, "mla_decode_absorbed_noalloc")


def _decode_checked_desc(q_nope, q_pe, kv_cache, cache_len, w_kv_b, *, n_splits, d_kv, softmax_scale, rope_base,
                         out_dtype, algo, return_lse, out, lse, workspace):
    """Checks every decode tensor (shapes, dtypes, layouts, device) and
    returns (descriptor, d_v)."""
    if q_nope.dim() != 3 or q_pe.dim() != 3 or kv_cache.dim() != 3 or w_kv_b.dim() != 2:
        raise ValueError("expected q_nope, q_pe [B,H,*], kv_cache [B,L_max,d_kv+d_rope], "
                         "w_kv_b [H*(d_nope+d_v), d_kv]")
    B, H, d_nope = q_nope.shape
    d_rope = q_pe.shape[-1]
    row = kv_cache.shape[-1]
    if d_kv is None:
        d_kv = row - d_rope
    if d_kv + d_rope != row:
        raise ValueError(f"kv_cache rows are {row} wide, expected d_kv + d_rope = {d_kv + d_rope}")
    if H < 1 or w_kv_b.shape[0] % H != 0 or w_kv_b.shape[0] // H <= d_nope:
        raise ValueError(f"w_kv_b rows ({w_kv_b.shape[0]}) must be H*(d_nope+d_v) with H={H}, d_nope={d_nope}")
    d_v = w_kv_b.shape[0] // H - d_nope
    dev = q_nope.device
    _expect(q_nope, "q_nope", (B, H, d_nope), q_nope.dtype, dev)
    _expect(q_pe, "q_pe", (B, H, d_rope), q_nope.dtype, dev)
    _expect(w_kv_b, "w_kv_b", (H * (d_nope + d_v), d_kv), q_nope.dtype, dev)
    _expect(cache_len, "cache_len", (B,), torch.int32, dev)
    if kv_cache.shape[0] != B:
        raise ValueError(f"kv_cache holds {kv_cache.shape[0]} sequences, expected {B}")
    if kv_cache.dtype != q_nope.dtype:
        raise ValueError(f"kv_cache has dtype {kv_cache.dtype}, expected {q_nope.dtype}")
    if kv_cache.device != dev:
        raise ValueError(f"kv_cache is on {kv_cache.device}, expected {dev}")
    if kv_cache.stride(-1) != 1 or kv_cache.stride(-2) != row or kv_cache.stride(0) < kv_cache.shape[1] * row:
        raise ValueError("kv_cache rows must be contiguous and sequences must not overlap")
    if out is not None:
        _expect(out, "out", (B, H, d_v), out_dtype, dev)
    if return_lse and lse is not None:
        _expect(lse, "lse", (B, H), torch.float32, dev)
    if workspace is not None:
        _expect_workspace(workspace, dev)
    _expect_cuda(dev)
    dt = _dtype_code(q_nope.dtype)
    desc = decode_desc(batch=B, n_heads=H, d_kv=d_kv, d_nope=d_nope, d_rope=d_rope, d_v=d_v,
                       max_cache_len=kv_cache.shape[1], cache_batch_stride=kv_cache.stride(0),
                       n_splits=n_splits, softmax_scale=softmax_scale, rope_base=rope_base, in_dtype=dt,
                       out_dtype=_dtype_code(out_dtype), algo=algo)
    return desc, d_v


def mla_timing_begin():
    _check(_lib().mla_timing_begin(), "mla_timing_begin")


def mla_timing_end():
    _check(_lib().mla_timing_end(), "mla_timing_end")


def mla_timing_reset():
    _check(_lib().mla_timing_reset(), "mla_timing_reset")


def mla_timing_get() -> dict:
    """{kernel name: (total ms, launches)} accumulated since the last reset."""
    lib = _lib()
    res = {}
    for i in range(lib.mla_timing_count()):
        name, ms, n = ctypes.c_char_p(), ctypes.c_double(), ctypes.c_int64()
        _check(lib.mla_timing_get(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(n)), "mla_timing_get")
        res[name.value.decode()] = (ms.value, n.value)
    return res


def build_info() -> str:
    return _lib().mla_build_info().decode()
