"""Python binding of the HIP library ``libfa.so`` (argument marshalling only).

The functions ``fa_fwd``, ``fa_fwd_f32``, ``fa_fwd_fp8``, ``fa_bwd``, ``fa_decode``,
``fa_decode_noalloc``, ``fa_decode_workgroups``,
``fa_decode_fp8``, ``fa_decode_fp8_workgroups``, ``fa_decode_int8``, ``fa_decode_int8_workgroups``,
``fa_read_probe``, ``fa_strerror`` and ``fa_release_workspace`` mirror the C entry points of
``include/fa.h`` one to one: pointers may be given as integers or as objects
with a ``data_ptr()`` method (torch tensors), streams as integers, None (the
default stream) or objects with a ``cuda_stream`` attribute.  A nonzero
status raises :class:`FAError`.

``attention`` and ``decode`` are conveniences for torch tensors: they check
dtypes/shapes/contiguity, allocate the outputs with torch and call the entry
points above.  Every step of the computation runs in the HIP kernels; if the
library is not built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_OK = 0
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_UNSUPPORTED",
                4: "FA_ERR_ALLOC", 5: "FA_ERR_LAUNCH", 6: "FA_ERR_DEVICE", 7: "FA_ERR_SCRATCH"}
DECODE_SCRATCH_BYTES = 4 << 20   # FA_DECODE_SCRATCH_BYTES of include/fa.h
STATUS_CODES = {v: k for k, v in STATUS_NAMES.items()}

_lib = None
_lock = threading.Lock()


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({fa_strerror(status)})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with "
                              "`python -m exact_tiled_attention_02_amd.build`")
        lib = ctypes.CDLL(path)
        P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.fa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, P]
        lib.fa_fwd.restype = I
        lib.fa_fwd_f32.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, P]
        lib.fa_fwd_f32.restype = I
        lib.fa_fwd_fp8.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P]
        lib.fa_fwd_fp8.restype = I
        lib.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P]
        lib.fa_bwd.restype = I
        lib.fa_decode.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P]
        lib.fa_decode.restype = I
        lib.fa_decode_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P]
        lib.fa_decode_noalloc.restype = I
        lib.fa_decode_workgroups.argtypes = [I, I, I, I, I, I]
        lib.fa_decode_workgroups.restype = I
        lib.fa_decode_fp8.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P]
        lib.fa_decode_fp8.restype = I
        lib.fa_decode_fp8_workgroups.argtypes = [I, I, I, I, I, I]
        lib.fa_decode_fp8_workgroups.restype = I
        lib.fa_decode_int8.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P]
        lib.fa_decode_int8.restype = I
        lib.fa_decode_int8_workgroups.argtypes = [I, I, I, I, I, I]
        lib.fa_decode_int8_workgroups.restype = I
        lib.fa_strerror.argtypes = [I]
        lib.fa_strerror.restype = ctypes.c_char_p
        lib.fa_read_probe.argtypes = [P, ctypes.c_size_t, P, P]
        lib.fa_read_probe.restype = I
        lib.fa_release_workspace.argtypes = []
        lib.fa_release_workspace.restype = None
        _lib = lib
        return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    dp = getattr(x, "data_ptr", None)
    if dp is not None:
        return dp()
    raise TypeError(f"cannot take a device pointer from {type(x).__name__}")


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    cs = getattr(s, "cuda_stream", None)
    if cs is not None:
        return cs
    raise TypeError(f"cannot take a stream handle from {type(s).__name__}")


def _check(st: int, where: str) -> None:
    if st != FA_OK:
        raise FAError(st, where)


# --- one-to-one entry points -------------------------------------------------

def _causal(c) -> int:
    """0 / False: no mask; 1 / True: top-left causal; 2: bottom-right causal."""
    if isinstance(c, bool):
        return int(c)
    if c == "bottom_right":
        return 2
    if c == "top_left":
        return 1
    return int(c)


def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale, stream=None) -> None:
    _check(load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Tq, Tk, d,
                         _causal(causal), float(scale), _stream(stream)), "fa_fwd")


def fa_fwd_f32(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale, stream=None) -> None:
    _check(load().fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Tq, Tk,
                             d, _causal(causal), float(scale), _stream(stream)), "fa_fwd_f32")


def fa_fwd_fp8(q, k, v, qscale, kscale, vscale, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale,
               stream=None) -> None:
    _check(load().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(qscale), _ptr(kscale), _ptr(vscale),
                             _ptr(o), _ptr(lse), B, Hq, Hkv, Tq, Tk, d, _causal(causal),
                             float(scale), _stream(stream)), "fa_fwd_fp8")


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Tq, Tk, d, causal, scale,
           stream=None) -> None:
    _check(load().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                         _ptr(dk), _ptr(dv), B, Hq, Hkv, Tq, Tk, d, _causal(causal),
                         float(scale), _stream(stream)), "fa_bwd")


def fa_decode(q, kcache, vcache, seqlens, o, B, Hq, Hkv, Tk_max, d, num_splits, stream=None) -> None:
    _check(load().fa_decode(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(seqlens), _ptr(o), B, Hq,
                            Hkv, Tk_max, d, int(num_splits), _stream(stream)), "fa_decode")


def fa_decode_noalloc(q, kcache, vcache, seqlens, o, B, Hq, Hkv, Tk_max, d, num_splits,
                      stream=None) -> None:
    _check(load().fa_decode_noalloc(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(seqlens), _ptr(o), B,
                                    Hq, Hkv, Tk_max, d, int(num_splits), _stream(stream)),
           "fa_decode_noalloc")


def fa_decode_workgroups(B, Hq, Hkv, Tk_max, d, num_splits) -> int:
    """Workgroup count fa_decode would use; raises FAError on a negative status."""
    n = load().fa_decode_workgroups(B, Hq, Hkv, Tk_max, d, int(num_splits))
    if n < 0:
        raise FAError(-n, "fa_decode_workgroups")
    return n


def fa_decode_fp8(q, kcache, vcache, kscale, vscale, seqlens, o, B, Hq, Hkv, Tk_max, d,
                  num_splits, stream=None) -> None:
    _check(load().fa_decode_fp8(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(kscale), _ptr(vscale),
                                _ptr(seqlens), _ptr(o), B, Hq, Hkv, Tk_max, d, int(num_splits),
                                _stream(stream)), "fa_decode_fp8")


def fa_decode_fp8_workgroups(B, Hq, Hkv, Tk_max, d, num_splits) -> int:
    n = load().fa_decode_fp8_workgroups(B, Hq, Hkv, Tk_max, d, int(num_splits))
    if n < 0:
        raise FAError(-n, "fa_decode_fp8_workgroups")
    return n


def fa_decode_int8(q, kcache, vcache, kscale, vscale, seqlens, o, B, Hq, Hkv, Tk_max, d,
                   num_splits, stream=None) -> None:
    _check(load().fa_decode_int8(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(kscale), _ptr(vscale),
                                 _ptr(seqlens), _ptr(o), B, Hq, Hkv, Tk_max, d, int(num_splits),
                                 _stream(stream)), "fa_decode_int8")


def fa_decode_int8_workgroups(B, Hq, Hkv, Tk_max, d, num_splits) -> int:
    n = load().fa_decode_int8_workgroups(B, Hq, Hkv, Tk_max, d, int(num_splits))
    if n < 0:
        raise FAError(-n, "fa_decode_int8_workgroups")
    return n


def fa_read_probe(src, nbytes, sink, stream=None) -> None:
    _check(load().fa_read_probe(_ptr(src), int(nbytes), _ptr(sink), _stream(stream)), "fa_read_probe")


def fa_strerror(status: int) -> str:
    return load().fa_strerror(int(status)).decode()


def fa_release_workspace() -> None:
    load().fa_release_workspace()


def prepared(entry: str, *args, stream=None):
    """Marshal the arguments of entry point `entry` once and return a
    zero-argument callable that makes the call (for timing loops: no
    per-call pointer extraction).  The callable raises FAError on a
    nonzero status."""
    lib = load()
    fn = getattr(lib, entry)
    conv = []
    for a, t in zip(args, fn.argtypes[:-1]):
        if t is ctypes.c_void_p:
            conv.append(_ptr(a))
        elif t is ctypes.c_float:
            conv.append(float(a))
        else:
            conv.append(int(a))
    conv.append(_stream(stream))
    cargs = [t(v) if v is not None else None for t, v in zip(fn.argtypes, conv)]

    def call():
        st = fn(*cargs)
        if st != FA_OK:
            raise FAError(st, entry)
    return call


# --- torch conveniences --------------------------------------------------------

def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def attention(q, k, v, *, causal: bool, scale: float | None = None, return_lse: bool = True,
              out=None, lse=None, stream=None):
    """softmax(q k^T * scale) v for contiguous [B,H,T,d] cuda tensors.

    bf16 inputs use ``fa_fwd``; fp32 inputs use ``fa_fwd_f32``.  Returns
    (o, lse) or o.
    """
    import torch
    _require(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k, v must be [B,H,T,d]")
    _require(q.is_cuda and k.is_cuda and v.is_cuda, "tensors must live on the GPU")
    _require(q.dtype == k.dtype == v.dtype and q.dtype in (torch.bfloat16, torch.float32),
             "q, k, v must all be bf16 or all fp32")
    _require(q.is_contiguous() and k.is_contiguous() and v.is_contiguous(), "tensors must be contiguous")
    B, Hq, Tq, d = q.shape
    Bk, Hkv, Tk, dk = k.shape
    _require(Bk == B and dk == d and tuple(v.shape) == tuple(k.shape), "shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    fn = fa_fwd if q.dtype == torch.bfloat16 else fa_fwd_f32
    fn(q, k, v, out, lse if return_lse else None, B, Hq, Hkv, Tq, Tk, d, causal, scale, stream)
    return (out, lse) if return_lse else out


def decode(q, kcache, vcache, seqlens, *, num_splits: int = 0, out=None, stream=None):
    """Single-query attention over a KV cache; q [B,Hq,d], caches [B,Hkv,Tmax,d] bf16,
    seqlens [B] int32 on the GPU."""
    import torch
    _require(q.dim() == 3 and kcache.dim() == 4 and vcache.shape == kcache.shape, "bad shapes")
    _require(q.dtype == kcache.dtype == vcache.dtype == torch.bfloat16, "decode takes bf16")
    _require(seqlens.dtype == torch.int32 and seqlens.is_cuda, "seqlens must be int32 on the GPU")
    _require(q.is_contiguous() and kcache.is_contiguous() and vcache.is_contiguous(),
             "tensors must be contiguous")
    B, Hq, d = q.shape
    _, Hkv, Tmax, _ = kcache.shape
    if out is None:
        out = torch.empty_like(q)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    fa_decode(q, kcache, vcache, seqlens, out, B, Hq, Hkv, Tmax, d, num_splits, stream)
    return out


def attention_backward(q, k, v, o, lse, dout, *, causal: bool, scale: float | None = None,
                       dq=None, dk=None, dv=None, stream=None):
    """Gradients (dq, dk, dv) of ``attention`` for bf16 [B,H,T,d] cuda tensors,
    from the forward's o and lse (``fa_bwd``)."""
    import torch
    _require(all(t.dim() == 4 and t.is_cuda and t.is_contiguous() and t.dtype == torch.bfloat16
                 for t in (q, k, v, o, dout)),
             "q, k, v, o, dout must be contiguous bf16 [B,H,T,d] cuda tensors")
    _require(lse.dtype == torch.float32 and lse.is_cuda and lse.is_contiguous(),
             "lse must be contiguous fp32 on the GPU")
    B, Hq, Tq, d = q.shape
    Bk, Hkv, Tk, dk_ = k.shape
    _require(Bk == B and dk_ == d and tuple(v.shape) == tuple(k.shape), "shape mismatch")
    _require(tuple(o.shape) == tuple(q.shape) == tuple(dout.shape), "o/dout shape mismatch")
    _require(tuple(lse.shape) == (B, Hq, Tq), "lse must be [B,Hq,Tq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Tq, Tk, d, causal, scale, stream)
    return dq, dk, dv


def decode_fp8(q, kcache, vcache, kscale, vscale, seqlens, *, num_splits: int = 0, out=None,
               stream=None):
    """Single-query attention over an E4M3 KV cache: q [B,Hq,d] bf16, caches
    [B,Hkv,Tmax,d] uint8 codes, scales [B,Hkv,Tmax] fp32, seqlens [B] int32."""
    return _decode_codes(fa_decode_fp8, q, kcache, vcache, kscale, vscale, seqlens, num_splits,
                         out, stream)


def decode_int8(q, kcache, vcache, kscale, vscale, seqlens, *, num_splits: int = 0, out=None,
                stream=None):
    """Single-query attention over an int8 KV cache: q [B,Hq,d] bf16, caches
    [B,Hkv,Tmax,d] int8 codes (torch int8 or their bytes as uint8), scales
    [B,Hkv,Tmax] fp32, seqlens [B] int32."""
    import torch
    if kcache.dtype == torch.int8:
        kcache = kcache.view(torch.uint8)
    if vcache.dtype == torch.int8:
        vcache = vcache.view(torch.uint8)
    return _decode_codes(fa_decode_int8, q, kcache, vcache, kscale, vscale, seqlens, num_splits,
                         out, stream)


def _decode_codes(entry, q, kcache, vcache, kscale, vscale, seqlens, num_splits, out, stream):
    import torch
    _require(q.dim() == 3 and kcache.dim() == 4 and vcache.shape == kcache.shape, "bad shapes")
    _require(q.dtype == torch.bfloat16 and kcache.dtype == vcache.dtype == torch.uint8,
             "q must be bf16 and the caches one-byte codes")
    _require(kscale.dtype == vscale.dtype == torch.float32 and
             tuple(kscale.shape) == tuple(vscale.shape) == tuple(kcache.shape[:3]),
             "scales must be fp32 [B,Hkv,Tmax]")
    _require(seqlens.dtype == torch.int32 and seqlens.is_cuda, "seqlens must be int32 on the GPU")
    _require(all(t.is_contiguous() for t in (q, kcache, vcache, kscale, vscale)),
             "tensors must be contiguous")
    B, Hq, d = q.shape
    _, Hkv, Tmax, _ = kcache.shape
    if out is None:
        out = torch.empty_like(q)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    entry(q, kcache, vcache, kscale, vscale, seqlens, out, B, Hq, Hkv, Tmax, d, num_splits, stream)
    return out
