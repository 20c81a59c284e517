"""Python binding of libfattn, the MI355X fused attention library (forward and backward).

Argument marshalling only: every step of the computation runs in the HIP kernels of
libfattn.so; torch supplies device memory and the current stream. Importing this package loads
the in-tree library and fails loudly if it has not been built.

    o, lse = attn_fwd(q, k, v, causal=True)      # q [B,Hq,Tq,d], k/v [B,Hkv,Tk,d] on the GPU
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, causal=True)
"""

from __future__ import annotations

import ctypes
import math
import os
import re
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
# FATTN_LIB names another build of the same library (the tests' host-only sanitizer build)
LIB_PATH = os.environ.get("FATTN_LIB") or os.path.join(_HERE, "libfattn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "fattn.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python io_aware_tiled_amd/build.py` first")

# torch is imported first so that its bundled HIP runtime is the one in the process: libfattn
# needs libamdhip64.so.7 by soname and then binds to that same runtime, which is the one that
# owns the streams and device pointers torch hands over. (Loaded the other way round, the
# system runtime and torch's bundled HSA runtime would be mixed in one process.)
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)


def _header_constants():
    consts = {}
    with open(HEADER_PATH) as f:
        for m in re.finditer(r"#define\s+(FATTN_\w+)\s+\(?(-?\d+)\)?", f.read()):
            consts[m.group(1)] = int(m.group(2))
    return consts


_C = _header_constants()
FATTN_OK = _C["FATTN_OK"]
FATTN_ERR_INVALID = _C["FATTN_ERR_INVALID"]
FATTN_ERR_UNSUPPORTED = _C["FATTN_ERR_UNSUPPORTED"]
FATTN_ERR_HIP = _C["FATTN_ERR_HIP"]
FATTN_ERR_NOMEM = _C["FATTN_ERR_NOMEM"]
FATTN_F32 = _C["FATTN_F32"]
FATTN_BF16 = _C["FATTN_BF16"]
FATTN_KERNEL_AUTO = _C["FATTN_KERNEL_AUTO"]
FATTN_KERNEL_PREFILL_MFMA = _C["FATTN_KERNEL_PREFILL_MFMA"]
FATTN_KERNEL_PREFILL_F32 = _C["FATTN_KERNEL_PREFILL_F32"]
FATTN_KERNEL_DECODE_SPLITK = _C["FATTN_KERNEL_DECODE_SPLITK"]


class FattnCfg(ctypes.Structure):
    """Mirror of fattn_cfg_t."""

    _fields_ = [(n, ctypes.c_int) for n in
                ("kernel", "block_q", "block_kv", "waves", "splits", "schedule")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_vp, _i, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
_FWD_ARGS = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp]
lib.attn_fwd.argtypes = _FWD_ARGS
lib.attn_fwd.restype = _i
lib.attn_fwd_cfg.argtypes = _FWD_ARGS + [ctypes.POINTER(FattnCfg)]
lib.attn_fwd_cfg.restype = _i
lib.attn_fwd_noalloc.argtypes = _FWD_ARGS
lib.attn_fwd_noalloc.restype = _i
lib.attn_fwd_window.argtypes = _FWD_ARGS
lib.attn_fwd_window.restype = _i
lib.attn_fwd_window_cfg.argtypes = _FWD_ARGS + [ctypes.POINTER(FattnCfg)]
lib.attn_fwd_window_cfg.restype = _i
lib.attn_fwd_varlen.argtypes = [_vp] * 7 + [_i] * 10 + [_f, _i, _vp]
lib.attn_bwd_varlen.argtypes = [_vp] * 11 + [_i] * 10 + [_f, _i, _vp]
lib.attn_bwd_varlen.restype = _i
lib.attn_fwd_varlen.restype = _i
lib.attn_fwd_paged.argtypes = [_vp] * 7 + [_i] * 7 + [_f, _i, _vp]
lib.attn_fwd_paged.restype = _i
lib.attn_bwd.argtypes = [_vp] * 9 + [_i] * 8 + [_f, _i, _vp]
lib.attn_bwd.restype = _i
lib.attn_fwd_plan.argtypes = [_i] * 8 + [ctypes.POINTER(FattnCfg), ctypes.POINTER(FattnCfg)]
lib.attn_fwd_plan.restype = _i
lib.fattn_strerror.argtypes = [_i]
lib.fattn_strerror.restype = ctypes.c_char_p
lib.fattn_last_error.argtypes = []
lib.fattn_last_error.restype = ctypes.c_char_p
lib.fattn_version.argtypes = []
lib.fattn_version.restype = _i
lib.fattn_release.argtypes = []
lib.fattn_release.restype = _i


class FattnError(RuntimeError):
    def __init__(self, code: int, detail: str = ""):
        msg = f"libfattn: {fattn_strerror(code)} (code {code})"
        super().__init__(msg + (f": {detail}" if detail else ""))
        self.code = code
        self.detail = detail


def fattn_last_error() -> str:
    """Why the calling thread's most recent library call failed ('' after a success)."""
    return lib.fattn_last_error().decode()


def fattn_strerror(code: int) -> str:
    return lib.fattn_strerror(int(code)).decode()


def fattn_version() -> int:
    return lib.fattn_version()


def fattn_release() -> None:
    rc = lib.fattn_release()
    if rc != FATTN_OK:
        raise FattnError(rc)


def check_out(name: str, t, shape, dtype, device) -> None:
    """A caller-supplied output buffer must be exactly what the kernels write into: the expected
    shape and dtype, contiguous, on the inputs' device. Raises ValueError (TypeError for the
    dtype) before anything is launched; the kernels would otherwise write past a short buffer
    or through a strided view."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")


def _make_cfg(cfg) -> Optional[FattnCfg]:
    if cfg is None:
        return None
    if isinstance(cfg, FattnCfg):
        return cfg
    c = FattnCfg()
    for k, v in dict(cfg).items():
        setattr(c, k, int(v))
    return c


def attn_fwd_plan(B, Hq, Hkv, Tq, Tk, d, causal, dtype, cfg=None) -> dict:
    """The launch configuration attn_fwd would use (host only, no GPU needed)."""
    out = FattnCfg()
    c = _make_cfg(cfg)
    rc = lib.attn_fwd_plan(B, Hq, Hkv, Tq, Tk, d, int(causal), dtype,
                           ctypes.byref(c) if c is not None else None, ctypes.byref(out))
    if rc != FATTN_OK:
        raise FattnError(rc, fattn_last_error())
    return out.as_dict()


def attn_fwd_raw(Q, K, V, O, LSE, B, Hq, Hkv, Tq, Tk, d, causal, scale, dtype, stream,
                 cfg=None, window=None) -> int:
    """The C call with plain integers for pointers; returns the library's status code.

    With ``window`` set, calls attn_fwd_window[_cfg] (causal implied; ``causal`` is ignored).
    """
    c = _make_cfg(cfg)
    if window is not None:
        if c is None:
            return lib.attn_fwd_window(Q, K, V, O, LSE, B, Hq, Hkv, Tq, Tk, d, int(window), scale,
                                       dtype, stream)
        return lib.attn_fwd_window_cfg(Q, K, V, O, LSE, B, Hq, Hkv, Tq, Tk, d, int(window),
                                       scale, dtype, stream, ctypes.byref(c))
    if c is None:
        return lib.attn_fwd(Q, K, V, O, LSE, B, Hq, Hkv, Tq, Tk, d, causal, scale, dtype, stream)
    return lib.attn_fwd_cfg(Q, K, V, O, LSE, B, Hq, Hkv, Tq, Tk, d, causal, scale, dtype, stream,
                            ctypes.byref(c))


def attn_fwd(q, k, v, causal: bool = False, scale: Optional[float] = None, out=None, lse=None,
             cfg=None, stream=None, window: Optional[int] = None) -> Tuple["object", "object"]:
    """Fused attention forward on torch GPU tensors; returns (o, lse).

    q: [B, Hq, Tq, d]; k, v: [B, Hkv, Tk, d]; contiguous, all float32 or all bfloat16, on the
    current device. o has q's dtype, lse is float32 [B, Hq, Tq] (natural log). scale defaults to
    1/sqrt(d). The call is enqueued on `stream` (default: torch's current stream).
    ``window`` (requires ``causal``): sliding-window attention, row at position p sees keys
    p - window < j <= p (attn_fwd_window).
    """
    import torch

    if window is not None and not causal:
        raise ValueError("a sliding window is a causal mask: pass causal=True")

    if q.dtype == torch.bfloat16:
        dtype = FATTN_BF16
    elif q.dtype == torch.float32:
        dtype = FATTN_F32
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, q has {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, T, d]")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, Hq, Tq, d = q.shape
    Bk, Hkv, Tk, dk = k.shape
    if (Bk, dk) != (B, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    check_out("out", out, q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    check_out("lse", lse, (B, Hq, Tq), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    rc = attn_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      B, Hq, Hkv, Tq, Tk, d, int(bool(causal)), float(scale), dtype, stream, cfg,
                      window)
    if rc != FATTN_OK:
        raise FattnError(rc, fattn_last_error())
    return out, lse


def attn_bwd_raw(Q, K, V, O, dO, LSE, dQ, dK, dV, B, Hq, Hkv, Tq, Tk, d, causal, window, scale,
                 dtype, stream) -> int:
    """The C call attn_bwd with plain integers for pointers; returns the library's status code."""
    return lib.attn_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, B, Hq, Hkv, Tq, Tk, d, causal, window,
                        scale, dtype, stream)


def attn_bwd(q, k, v, o, lse, do, causal: bool = False, scale: Optional[float] = None,
             window: Optional[int] = None, dq=None, dk=None, dv=None, stream=None):
    """Backward of attn_fwd on torch GPU tensors; returns (dq, dk, dv).

    q, o, do: [B, Hq, Tq, d]; k, v: [B, Hkv, Tk, d]; bfloat16, contiguous, on the current
    device; lse: float32 [B, Hq, Tq] from the forward call with the same causal, window and
    scale (default 1/sqrt(d)). Enqueued on `stream` (default: torch's current stream).
    """
    import torch

    if window is not None and not causal:
        raise ValueError("a sliding window is a causal mask: pass causal=True")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("lse", lse)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, Hq, Tq, d = q.shape
    Bk, Hkv, Tk, dk_ = k.shape
    if (Bk, dk_) != (B, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if tuple(o.shape) != tuple(q.shape) or tuple(do.shape) != tuple(q.shape):
        raise ValueError("o and do must have q's shape")
    if tuple(lse.shape) != (B, Hq, Tq):
        raise ValueError("lse must be [B, Hq, Tq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        check_out(name, t, ref.shape, torch.bfloat16, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    rc = attn_bwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                      lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Tq,
                      Tk, d, int(bool(causal)), int(window or 0), float(scale), FATTN_BF16, stream)
    if rc != FATTN_OK:
        raise FattnError(rc, fattn_last_error())
    return dq, dk, dv


def attn_fwd_paged_raw(Q, K_cache, V_cache, block_table, seq_lens, O, LSE, B, Hq, Hkv, d,
                       num_blocks, block_size, max_blocks_per_seq, scale, dtype, stream) -> int:
    """The C call attn_fwd_paged with plain integers for pointers; returns the status code."""
    return lib.attn_fwd_paged(Q, K_cache, V_cache, block_table, seq_lens, O, LSE, B, Hq, Hkv, d,
                              num_blocks, block_size, max_blocks_per_seq, scale, dtype, stream)


def attn_fwd_paged(q, k_cache, v_cache, block_table, seq_lens, scale: Optional[float] = None,
                   out=None, lse=None, stream=None):
    """One decode step over a paged KV cache; returns (o [B, Hq, d], lse [B, Hq]).

    q: [B, Hq, d] bfloat16; k_cache, v_cache: [num_blocks, Hkv, block_size, d] bfloat16;
    block_table: [B, max_blocks] int32; seq_lens: [B] int32; all contiguous on the current device.
    """
    import torch

    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    for name, t in (("block_table", block_table), ("seq_lens", seq_lens)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32, got {t.dtype}")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_table", block_table), ("seq_lens", seq_lens)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 3 or k_cache.dim() != 4 or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q must be [B, Hq, d], k_cache and v_cache [num_blocks, Hkv, bs, d]")
    B, Hq, d = q.shape
    num_blocks, Hkv, bs, dk_ = k_cache.shape
    if dk_ != d:
        raise ValueError("head dims differ")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_blocks] and seq_lens [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    check_out("out", out, q.shape, torch.bfloat16, q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    check_out("lse", lse, (B, Hq), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    rc = attn_fwd_paged_raw(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                            block_table.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
                            lse.data_ptr(), B, Hq, Hkv, d, num_blocks, bs, block_table.shape[1],
                            float(scale), FATTN_BF16, stream)
    if rc != FATTN_OK:
        raise FattnError(rc, fattn_last_error())
    return out, lse


def attn_fwd_varlen_raw(Q, K, V, O, LSE, cu_q, cu_k, num_seqs, total_q, total_k, max_q, max_k,
                        Hq, Hkv, d, causal, window, scale, dtype, stream) -> int:
    """The C call attn_fwd_varlen with plain integers for pointers; returns the status code."""
    return lib.attn_fwd_varlen(Q, K, V, O, LSE, cu_q, cu_k, num_seqs, total_q, total_k, max_q,
                               max_k, Hq, Hkv, d, causal, window, scale, dtype, stream)


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    causal: bool = False, scale: Optional[float] = None,
                    window: Optional[int] = None, out=None, lse=None, stream=None):
    """Attention over a packed batch; returns (o [total_q, Hq, d], lse [Hq, total_q]).

    q: [total_q, Hq, d]; k, v: [total_k, Hkv, d]; bfloat16, contiguous, on the current device.
    cu_seqlens_q / cu_seqlens_k: int32 [num_seqs + 1] cumulative lengths on the device.
    """
    import torch

    if window is not None and not causal:
        raise ValueError("a sliding window is a causal mask: pass causal=True")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
        if t.dim() != 3:
            raise ValueError(f"{name} must be [total, H, d]")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or t.dim() != 1:
            raise TypeError(f"{name} must be a 1-D int32 tensor")
    for name, t in (("q", q), ("k", k), ("v", v), ("cu_seqlens_q", cu_seqlens_q),
                    ("cu_seqlens_k", cu_seqlens_k)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    total_q, Hq, d = q.shape
    total_k, Hkv, dk_ = k.shape
    if dk_ != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [total_k, Hkv, d] with q's d")
    num_seqs = cu_seqlens_q.shape[0] - 1
    if cu_seqlens_k.shape[0] != num_seqs + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    check_out("out", out, q.shape, torch.bfloat16, q.device)
    if lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    check_out("lse", lse, (Hq, total_q), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    rc = attn_fwd_varlen_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(),
                             max(num_seqs, 0), total_q, total_k, int(max_seqlen_q),
                             int(max_seqlen_k), Hq, Hkv, d, int(bool(causal)), int(window or 0),
                             float(scale), FATTN_BF16, stream)
    if rc != FATTN_OK:
        raise FattnError(rc, fattn_last_error())
    return out, lse


def attn_bwd_varlen_raw(Q, K, V, O, dO, LSE, dQ, dK, dV, cu_q, cu_k, num_seqs, total_q, total_k,
                        max_q, max_k, Hq, Hkv, d, causal, window, scale, dtype, stream) -> int:
    """The C call attn_bwd_varlen with plain integers for pointers; returns the status code."""
    return lib.attn_bwd_varlen(Q, K, V, O, dO, LSE, dQ, dK, dV, cu_q, cu_k, num_seqs, total_q,
                               total_k, max_q, max_k, Hq, Hkv, d, causal, window, scale, dtype,
                               stream)


def attn_bwd_varlen(q, k, v, o, lse, do, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                    max_seqlen_k: int, causal: bool = False, scale: Optional[float] = None,
                    window: Optional[int] = None, dq=None, dk=None, dv=None, stream=None):
    """Backward of attn_fwd_varlen; returns (dq, dk, dv) in the packed layouts.

    q, o, do: [total_q, Hq, d]; k, v: [total_k, Hkv, d]; bfloat16; lse: float32 [Hq, total_q]
    from the forward call with the same offsets, causal, window and scale.
    """
    import torch

    if window is not None and not causal:
        raise ValueError("a sliding window is a causal mask: pass causal=True")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
        if t.dim() != 3:
            raise ValueError(f"{name} must be [total, H, d]")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or t.dim() != 1:
            raise TypeError(f"{name} must be a 1-D int32 tensor")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("lse", lse),
                    ("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    total_q, Hq, d = q.shape
    total_k, Hkv, dk_ = k.shape
    if dk_ != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [total_k, Hkv, d] with q's d")
    if tuple(o.shape) != tuple(q.shape) or tuple(do.shape) != tuple(q.shape):
        raise ValueError("o and do must have q's shape")
    if tuple(lse.shape) != (Hq, total_q):
        raise ValueError("lse must be [Hq, total_q]")
    num_seqs = cu_seqlens_q.shape[0] - 1
    if cu_seqlens_k.shape[0] != num_seqs + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        check_out(name, t, ref.shape, torch.bfloat16, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    rc = attn_bwd_varlen_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                             dv.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(),
                             max(num_seqs, 0), total_q, total_k, int(max_seqlen_q),
                             int(max_seqlen_k), Hq, Hkv, d, int(bool(causal)), int(window or 0),
                             float(scale), FATTN_BF16, stream)
    if rc != FATTN_OK:
        raise FattnError(rc, fattn_last_error())
    return dq, dk, dv
