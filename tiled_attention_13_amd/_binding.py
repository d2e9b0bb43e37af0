"""ctypes binding of ``libfa.so`` (the C ABI in ``include/fa.h``).

Argument marshalling only: tensors are passed as raw device pointers with
the current torch stream; every step of the forward and backward passes
runs in the HIP kernels.  There is no fallback: if the library is missing or the call fails,
an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
_lib = None

FA_F32, FA_BF16, FA_FP8_E4M3, FA_FP8_E4M3_PV = 0, 1, 2, 3
DTYPE_CODES = {"f32": FA_F32, "bf16": FA_BF16, "fp8": FA_FP8_E4M3, "fp8pv": FA_FP8_E4M3_PV}

# (name, restype, argtypes) of every entry point declared in include/fa.h
_P, _I64, _I, _F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
SIGNATURES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I, _F, _I, _P]),
    "fa_quant_fp8_e4m3": (_I, [_P, _P, _P, _I64, _I64, _I64, _P]),
    "fa_quant_v_pow2": (_I, [_P, _P, _P, _I64, _I64, _I64, _P]),
    "fa_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I, _F, _P]),
    "fa_fwd_partial": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I, _F, _P]),
    "fa_merge": (_I, [_P, _P, _I64, _P, _P, _I64, _I64, _I64, _I64, _P]),
    "fa_fwd_splitkv": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I, _F, _I64, _P]),
    "fa_fwd_splitkv_noalloc": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I, _F, _I64, _P]),
    "fa_fwd_blocksparse": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _I64, _I, _F, _P]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I, _F, _I, _P]),
    "fa_status_string": (ctypes.c_char_p, [_I]),
    "fa_abi_version": (_I, []),
}


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed with status {status}: {status_string(status)}")


def lib_path() -> str:
    return _LIB_PATH


def load_library(path: str):
    """Open a build of the C ABI at `path` with the signatures of include/fa.h."""
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(run `python -m tiled_attention_13_amd.build`)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load():
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load_library(_LIB_PATH)
    return _lib


def status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise FAError(status, where)


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _check_qkv(q, k, v, torch_dtype):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dtype != torch_dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {torch_dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [B, H, N, d]")
        if t.dim() != 4 or t.shape != q.shape:
            raise ValueError("q, k, v must share one [B, H, N, d] shape")
        if t.device != q.device:
            raise ValueError("q, k, v must be on one device")


def _check_out(name, t, shape, dtype, device):
    """A caller-supplied output must be exactly what the kernels write: the
    expected shape and dtype, contiguous, on the inputs' device (a smaller or
    differently typed buffer would be written past its end)."""
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fwd(q, k, v, causal: bool = False, softmax_scale: float | None = None, dtype: str | None = None,
        out=None, lse=None, with_lse: bool = True, stream=None):
    """Fused attention forward through ``fa_fwd``.

    q, k, v: contiguous device tensors ``[B, H, N, d]`` (float32 for
    dtype "f32", bfloat16 for "bf16", "fp8" and "fp8pv"; "fp8" quantises Q
    and K to e4m3 per 64-row tile inside the call, "fp8pv" also V, and runs
    P*V on e4m3 as well).  ``softmax_scale`` defaults to
    ``1/sqrt(d)``.  Returns ``(o, lse)`` (lse is None when ``with_lse`` is
    False and no ``lse`` buffer is given).
    """
    import torch
    if dtype is None:
        dtype = "f32" if q.dtype == torch.float32 else "bf16"
    code = DTYPE_CODES[dtype]
    _check_qkv(q, k, v, torch.float32 if dtype == "f32" else torch.bfloat16)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out("out", out, q.shape, q.dtype, q.device)
    if lse is None and with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_out("lse", lse, (B, H, N), torch.float32, q.device)
    st = load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
                       int(bool(causal)), scale, code, _stream_ptr(stream))
    _check(st, "fa_fwd")
    return out, lse


def quant_fp8(x, stream=None):
    """Per-64-row-tile e4m3fn quantisation of a bf16 ``[B, H, N, d]`` tensor.

    Returns ``(codes uint8 [B,H,N,d], scale float32 [B,H,ceil(N/64)])``.
    """
    import torch
    if not x.is_cuda or x.dtype != torch.bfloat16 or not x.is_contiguous() or x.dim() != 4:
        raise ValueError("x must be a contiguous bf16 device tensor [B, H, N, d]")
    B, H, N, d = x.shape
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scale = torch.empty((B, H, (N + 63) // 64), dtype=torch.float32, device=x.device)
    st = load().fa_quant_fp8_e4m3(_ptr(x), _ptr(codes), _ptr(scale), B * H, N, d, _stream_ptr(stream))
    _check(st, "fa_quant_fp8_e4m3")
    return codes, scale


def fwd_fp8(q8, q_scale, k8, k_scale, v, causal: bool = False, softmax_scale: float | None = None,
            out=None, lse=None, with_lse: bool = True, stream=None):
    """Attention forward on pre-quantised e4m3 Q/K (``fa_fwd_fp8``); V and O bf16."""
    import torch
    B, H, N, d = v.shape
    for name, t, dt in (("q8", q8, torch.uint8), ("k8", k8, torch.uint8), ("v", v, torch.bfloat16),
                        ("q_scale", q_scale, torch.float32), ("k_scale", k_scale, torch.float32)):
        if not t.is_cuda or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} device tensor")
    if q8.shape != v.shape or k8.shape != v.shape:
        raise ValueError("q8, k8, v must share one [B, H, N, d] shape")
    if q_scale.shape != (B, H, (N + 63) // 64) or k_scale.shape != q_scale.shape:
        raise ValueError("scales must be [B, H, ceil(N/64)]")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if q8.device != v.device or k8.device != v.device or q_scale.device != v.device or k_scale.device != v.device:
        raise ValueError("q8, k8, scales and v must be on one device")
    if out is None:
        out = torch.empty_like(v)
    else:
        _check_out("out", out, v.shape, torch.bfloat16, v.device)
    if lse is None and with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=v.device)
    elif lse is not None:
        _check_out("lse", lse, (B, H, N), torch.float32, v.device)
    st = load().fa_fwd_fp8(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v), _ptr(out), _ptr(lse),
                           B, H, N, d, int(bool(causal)), scale, _stream_ptr(stream))
    _check(st, "fa_fwd_fp8")
    return out, lse


def bwd(q, k, v, o, dout, lse, causal: bool = False, softmax_scale: float | None = None,
        dq=None, dk=None, dv=None, stream=None):
    """Gradient of the attention forward through ``fa_bwd`` (bf16 only).

    q, k, v, o, dout: contiguous bf16 device tensors ``[B, H, N, d]`` (o and
    lse as returned by ``fwd`` for the same q, k, v, causal and scale).
    Returns ``(dq, dk, dv)`` in bf16.
    """
    import torch
    _check_qkv(q, k, v, torch.bfloat16)
    for name, t in (("o", o), ("dout", dout)):
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous() or t.shape != q.shape:
            raise ValueError(f"{name} must be a contiguous bf16 device tensor shaped like q")
    B, H, N, d = q.shape
    if lse is None or not lse.is_cuda or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be the float32 [B, H, N] device tensor written by fwd")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    for name, t in (("o", o), ("dout", dout), ("lse", lse)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}")
    grads = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty_like(q)
        else:
            _check_out(name, t, q.shape, torch.bfloat16, q.device)
        grads.append(t)
    dq, dk, dv = grads
    st = load().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                       B, H, N, d, int(bool(causal)), scale, FA_BF16, _stream_ptr(stream))
    _check(st, "fa_bwd")
    return dq, dk, dv


def fwd_partial(q, k, v, kv_begin: int, kv_end: int, causal: bool = False, softmax_scale: float | None = None,
                o_part=None, lse_part=None, stream=None):
    """Attention over keys [kv_begin, kv_end) only (``fa_fwd_partial``), bf16 in.

    Returns ``(o_part float32 [B,H,N,d], lse_part float32 [B,H,N])``: O
    normalised over the range's visible keys and the range's logsumexp
    (-inf for rows that see none of them).
    """
    import torch
    _check_qkv(q, k, v, torch.bfloat16)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if o_part is None:
        o_part = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    else:
        _check_out("o_part", o_part, q.shape, torch.float32, q.device)
    if lse_part is None:
        lse_part = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_out("lse_part", lse_part, (B, H, N), torch.float32, q.device)
    st = load().fa_fwd_partial(_ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part), B, H, N, d,
                               int(kv_begin), int(kv_end), int(bool(causal)), scale, _stream_ptr(stream))
    _check(st, "fa_fwd_partial")
    return o_part, lse_part


def merge(o_parts, lse_parts, out=None, lse=None, with_lse: bool = True, stream=None):
    """Combine partial results (``fa_merge``): ``o_parts`` float32 [G,B,H,N,d],
    ``lse_parts`` float32 [G,B,H,N] -> (bf16 O [B,H,N,d], float32 lse [B,H,N])."""
    import torch
    if o_parts.dim() != 5 or o_parts.dtype != torch.float32 or not o_parts.is_contiguous() or not o_parts.is_cuda:
        raise ValueError("o_parts must be a contiguous float32 device tensor [G, B, H, N, d]")
    G, B, H, N, d = o_parts.shape
    _check_out("lse_parts", lse_parts, (G, B, H, N), torch.float32, o_parts.device)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=o_parts.device)
    else:
        _check_out("out", out, (B, H, N, d), torch.bfloat16, o_parts.device)
    if lse is None and with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=o_parts.device)
    elif lse is not None:
        _check_out("lse", lse, (B, H, N), torch.float32, o_parts.device)
    st = load().fa_merge(_ptr(o_parts), _ptr(lse_parts), G, _ptr(out), _ptr(lse), B, H, N, d, _stream_ptr(stream))
    _check(st, "fa_merge")
    return out, lse


def fwd_splitkv(q, k, v, n_splits: int, causal: bool = False, softmax_scale: float | None = None,
                out=None, lse=None, with_lse: bool = True, stream=None):
    """bf16 attention forward with the keys split into ``n_splits`` ranges run as
    separate workgroups and merged (``fa_fwd_splitkv``).  Returns ``(o, lse)``."""
    import torch
    _check_qkv(q, k, v, torch.bfloat16)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out("out", out, q.shape, torch.bfloat16, q.device)
    if lse is None and with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_out("lse", lse, (B, H, N), torch.float32, q.device)
    st = load().fa_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
                               int(bool(causal)), scale, int(n_splits), _stream_ptr(stream))
    _check(st, "fa_fwd_splitkv")
    return out, lse


def fwd_splitkv_noalloc(q, k, v, n_splits: int, out, lse=None, causal: bool = False,
                        softmax_scale: float | None = None, stream=None):
    """``fa_fwd_splitkv_noalloc``: the split-KV forward with its partial results
    in the library's static device buffer, so the call allocates nothing (for
    graph capture or loops that must not allocate).  The caller passes ``out``
    (bf16 like q) and optionally ``lse`` (float32 [B, H, N]); calls that overlap
    on one GPU race on the shared buffer.  Returns ``(out, lse)``."""
    import torch
    _check_qkv(q, k, v, torch.bfloat16)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    _check_out("out", out, q.shape, torch.bfloat16, q.device)
    if lse is not None:
        _check_out("lse", lse, (B, H, N), torch.float32, q.device)
    st = load().fa_fwd_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
                                       int(bool(causal)), scale, int(n_splits), _stream_ptr(stream))
    _check(st, "fa_fwd_splitkv_noalloc")
    return out, lse


def fwd_blocksparse(q, k, v, block_mask, causal: bool = False, softmax_scale: float | None = None,
                    out=None, lse=None, with_lse: bool = True, stream=None):
    """bf16 attention with a 64x64 block table (``fa_fwd_blocksparse``).

    ``block_mask``: uint8 device tensor ``[nb, nb]`` (shared by all heads) or
    ``[B, H, nb, nb]``, nb = ceil(N/64); nonzero = the block is computed.
    Returns ``(o, lse)``; rows that see no key get O = 0 and lse = -inf.
    """
    import torch
    _check_qkv(q, k, v, torch.bfloat16)
    B, H, N, d = q.shape
    nb = (N + 63) // 64
    if block_mask.dtype != torch.uint8 or block_mask.device != q.device or not block_mask.is_contiguous():
        raise ValueError("block_mask must be a contiguous uint8 device tensor")
    if tuple(block_mask.shape) == (nb, nb):
        stride = 0
    elif tuple(block_mask.shape) == (B, H, nb, nb):
        stride = nb * nb
    else:
        raise ValueError(f"block_mask must be [{nb}, {nb}] or [{B}, {H}, {nb}, {nb}]")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out("out", out, q.shape, torch.bfloat16, q.device)
    if lse is None and with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_out("lse", lse, (B, H, N), torch.float32, q.device)
    st = load().fa_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, _ptr(block_mask),
                                   stride, int(bool(causal)), scale, _stream_ptr(stream))
    _check(st, "fa_fwd_blocksparse")
    return out, lse


def quant_v_pow2(v, stream=None):
    """Power-of-two e4m3 quantisation of a bf16 V ``[B, H, N, d]`` (``fa_quant_v_pow2``).

    Returns ``(codes uint8 [B,H,d,np] (tile-permuted keys), scale_bytes uint8 [B,H,ceil(N/64),d])``.
    """
    import torch
    if not v.is_cuda or v.dtype != torch.bfloat16 or not v.is_contiguous() or v.dim() != 4:
        raise ValueError("v must be a contiguous bf16 device tensor [B, H, N, d]")
    B, H, N, d = v.shape
    np_ = (N + 63) // 64 * 64
    codes = torch.empty((B, H, d, np_), dtype=torch.uint8, device=v.device)
    sc = torch.empty((B, H, (N + 63) // 64, d), dtype=torch.uint8, device=v.device)
    st = load().fa_quant_v_pow2(_ptr(v), _ptr(codes), _ptr(sc), B * H, N, d, _stream_ptr(stream))
    _check(st, "fa_quant_v_pow2")
    return codes, sc
