"""Thin ctypes binding of libfa355.so (fused exact attention for gfx950) and of
the unfused comparator's libfa355_unfused.so.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their device pointers and torch's current HIP stream are passed to
the C ABI, and every step of the computation runs in the library's kernels.
PyTorch only supplies device memory and the stream. There is no fallback: if
the library cannot be loaded, every call raises.

The functions ``fa_fwd``, ``fa_fwd_persistent``, ``fa_fwd_kernel_name``, ``fa_bwd``,
``fa_bwd_noalloc``,
``fa_bwd_kernel_name``, ``fa_bwd_workspace_bytes``,
``fa_unfused_fwd``, ``fa_unfused_workspace_bytes``, ``fa_fa1_fwd``,
``fa_fa1_workspace_bytes``, ``fa_decode_fwd``,
``fa_decode_workspace_bytes`` and ``fa_strerror`` are the raw C entry points
(ctypes). ``fwd`` / ``bwd`` / ``unfused_fwd`` / ``fa1_fwd`` / ``decode_fwd`` are
tensor-level wrappers with the same semantics (``fwd_persistent`` for the
persistent comparator). ``attention`` wraps ``fwd`` and ``bwd`` as one
autograd operation.
"""
from __future__ import annotations

import ctypes
import math
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa355.so")
# The unfused comparator (rocBLAS GEMMs) is a library of its own, opened only
# when one of its entry points is called.
_LIB_UNFUSED_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                 "libfa355_unfused.so")

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_HEADDIM, FA_ERR_SCALE, FA_ERR_ALIGN, \
    FA_ERR_WORKSPACE, FA_ERR_HIP, FA_ERR_BLAS, FA_ERR_TOO_LARGE = range(10)
FA_BWD_NOALLOC_MAX_ROWS = 4194304


class FAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: error {code}: {strerror(code)}")


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python -m exact_io_aware_12_amd.build` "
            "(there is no CPU fallback)")
    # torch first, so the library binds to the HIP runtime torch already
    # mapped (both carry the soname libamdhip64.so.7) and streams/pointers are
    # shared.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def load_build(path: str):
    """Another build of libfa355.so (for instance the race-check build
    libfa355_strict.so next to it), with the same C signatures."""
    _load()   # torch's HIP runtime and the main library first
    return _bind(ctypes.CDLL(path))


def _bind(lib):
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_persistent.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_fwd_persistent.restype = i
    lib.fa_fwd_kernel_name.argtypes = [i, i, i, i, i]
    lib.fa_fwd_kernel_name.restype = ctypes.c_char_p
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_kernel_name.argtypes = [i, i, i, i, i]
    lib.fa_bwd_kernel_name.restype = ctypes.c_char_p
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_fa1_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_fa1_workspace_bytes.restype = sz
    lib.fa_fa1_fwd.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, vp]
    lib.fa_fa1_fwd.restype = i
    lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_decode_workspace_bytes.restype = sz
    lib.fa_decode_fwd.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, vp]
    lib.fa_decode_fwd.restype = i
    lib.fa_strerror.argtypes = [i]
    lib.fa_strerror.restype = ctypes.c_char_p
    return lib


_lib_unfused = None


def _load_unfused():
    global _lib_unfused
    if _lib_unfused is not None:
        return _lib_unfused
    _load()   # the fused library (and torch's HIP runtime) first
    if not os.path.exists(_LIB_UNFUSED_PATH):
        raise ImportError(f"{_LIB_UNFUSED_PATH} is missing: build it with "
                          "`python -m exact_io_aware_12_amd.build`")
    lib = ctypes.CDLL(_LIB_UNFUSED_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_unfused_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_unfused_workspace_bytes.restype = sz
    lib.fa_unfused_fwd.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, vp]
    lib.fa_unfused_fwd.restype = i
    _lib_unfused = lib
    return lib


def library():
    """The loaded ctypes library (raises if it is missing)."""
    return _load()


def library_unfused():
    """The unfused comparator's ctypes library (raises if it is missing)."""
    return _load_unfused()


# ----------------------------------------------------------------- raw C ABI
def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream) -> int:
    return _load().fa_fwd(q, k, v, o, lse, B, H, N, d, scale, int(causal), stream)


def fa_fwd_persistent(q, k, v, o, lse, B, H, N, d, scale, causal, stream) -> int:
    return _load().fa_fwd_persistent(q, k, v, o, lse, B, H, N, d, scale, int(causal), stream)


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
           scale, causal, stream) -> int:
    return _load().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes,
                          B, H, N, d, scale, int(causal), stream)


def fa_fwd_kernel_name(B, H, N, d, causal) -> str | None:
    """Name of the kernel fa_fwd launches for this shape (None if invalid)."""
    r = _load().fa_fwd_kernel_name(B, H, N, d, int(bool(causal)))
    return r.decode() if r is not None else None


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal,
                   stream) -> int:
    return _load().fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale,
                                  int(causal), stream)


def fa_bwd_kernel_name(B, H, N, d, causal) -> str | None:
    """Names of the kernels fa_bwd launches for this shape (None if invalid)."""
    r = _load().fa_bwd_kernel_name(B, H, N, d, int(bool(causal)))
    return r.decode() if r is not None else None


def fa_bwd_workspace_bytes(B, H, N, d) -> int:
    return _load().fa_bwd_workspace_bytes(B, H, N, d)


def fa_unfused_fwd(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, scale, causal,
                   stream) -> int:
    return _load_unfused().fa_unfused_fwd(q, k, v, o, lse, workspace, workspace_bytes, B, H,
                                          N, d, scale, int(causal), stream)


def fa_unfused_workspace_bytes(B, H, N, d) -> int:
    return _load_unfused().fa_unfused_workspace_bytes(B, H, N, d)


def fa_fa1_fwd(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, scale, causal,
               stream) -> int:
    return _load().fa_fa1_fwd(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d,
                              float(scale), int(bool(causal)), stream)


def fa_fa1_workspace_bytes(B, H, N, d) -> int:
    return _load().fa_fa1_workspace_bytes(B, H, N, d)


def fa_decode_fwd(q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, d, scale, causal,
                  stream) -> int:
    return _load().fa_decode_fwd(q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, d,
                                 scale, int(causal), stream)


def fa_decode_workspace_bytes(B, H, Nq, Nk, d) -> int:
    return _load().fa_decode_workspace_bytes(B, H, Nq, Nk, d)


def fa_strerror(code: int) -> str:
    return _load().fa_strerror(code).decode()


def strerror(code: int) -> str:
    try:
        return fa_strerror(code)
    except ImportError:
        return "library not loaded"


# ----------------------------------------------------------------- tensors
def _check(t, name, shape=None, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream_ptr(device, stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def fwd(q, k, v, *, causal: bool = False, scale: float | None = None, out=None, lse=None,
        stream=None):
    """O, LSE = attention(q, k, v): bf16 [B,H,N,d] in, bf16 O and fp32 LSE out."""
    return _fwd_call(fa_fwd, "fa_fwd", q, k, v, causal, scale, out, lse, stream)


def fwd_persistent(q, k, v, *, causal: bool = False, scale: float | None = None, out=None,
                   lse=None, stream=None):
    """The same O, LSE as ``fwd`` on a persistent grid (at most two resident
    workgroups per CU looping over the query tiles in a static snake order):
    the measured scheduling comparator of the fused pass."""
    return _fwd_call(fa_fwd_persistent, "fa_fwd_persistent", q, k, v, causal, scale, out, lse,
                     stream)


def _fwd_call(raw, name, q, k, v, causal, scale, out, lse, stream):
    import torch
    _check(q, "q", dtype=torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    _check(k, "k", q.shape, torch.bfloat16)
    _check(v, "v", q.shape, torch.bfloat16)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    _check(out, "out", q.shape, torch.bfloat16)
    _check(lse, "lse", (B, H, N), torch.float32)
    rc = raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
             B, H, N, d, float(scale), causal, _stream_ptr(q.device, stream))
    if rc != FA_OK:
        raise FAError(rc, name)
    return out, lse


def bwd(q, k, v, o, do, lse, *, causal: bool = False, scale: float | None = None,
        workspace=None, dq=None, dk=None, dv=None, stream=None):
    """dQ, dK, dV of sum(O * dO) for O = fwd(q, k, v)."""
    import torch
    _check(q, "q", dtype=torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check(t, n, q.shape, torch.bfloat16)
    _check(lse, "lse", (B, H, N), torch.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    _check(workspace, "workspace")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, n, q.shape, torch.bfloat16)
    rc = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                B, H, N, d, float(scale), causal, _stream_ptr(q.device, stream))
    if rc != FA_OK:
        raise FAError(rc, "fa_bwd")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, do, lse, *, causal: bool = False, scale: float | None = None,
                dq, dk, dv, stream=None):
    """``bwd`` through fa_bwd_noalloc: the caller passes the outputs; the
    library's static scratch replaces the workspace (nothing is allocated)."""
    import torch
    _check(q, "q", dtype=torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (do, "do"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, n, q.shape, torch.bfloat16)
    _check(lse, "lse", (B, H, N), torch.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rc = fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                        B, H, N, d, float(scale), causal, _stream_ptr(q.device, stream))
    if rc != FA_OK:
        raise FAError(rc, "fa_bwd_noalloc")
    return dq, dk, dv


def _fwd_with_workspace(q, k, v, causal, scale, out, lse, workspace, stream, raw, ws_bytes,
                        name):
    import torch
    _check(q, "q", dtype=torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    _check(k, "k", q.shape, torch.bfloat16)
    _check(v, "v", q.shape, torch.bfloat16)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    _check(out, "out", q.shape, torch.bfloat16)
    _check(lse, "lse", (B, H, N), torch.float32)
    need = ws_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    _check(workspace, "workspace")
    rc = raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
             workspace.data_ptr(), workspace.numel() * workspace.element_size(), B, H, N, d,
             float(scale), causal, _stream_ptr(q.device, stream))
    if rc != FA_OK:
        raise FAError(rc, name)
    return out, lse


def unfused_fwd(q, k, v, *, causal: bool = False, scale: float | None = None, out=None,
                lse=None, workspace=None, stream=None):
    """The same O, LSE as ``fwd`` by the unfused three-step method (S and P in
    device memory): the measured comparator of the fused pass."""
    return _fwd_with_workspace(q, k, v, causal, scale, out, lse, workspace, stream,
                               fa_unfused_fwd, fa_unfused_workspace_bytes, "fa_unfused_fwd")


def fa1_fwd(q, k, v, *, causal: bool = False, scale: float | None = None, out=None,
            lse=None, workspace=None, stream=None):
    """The same O, LSE as ``fwd`` with the loop order swapped (outer loop over
    key/value tiles, one workgroup per head, running state in device memory):
    the measured loop-order comparator of the fused pass."""
    return _fwd_with_workspace(q, k, v, causal, scale, out, lse, workspace, stream,
                               fa_fa1_fwd, fa_fa1_workspace_bytes, "fa_fa1_fwd")


def decode_fwd(q, k, v, *, causal: bool = False, scale: float | None = None, out=None,
               lse=None, workspace=None, stream=None):
    """O, LSE of Nq <= 32 query rows ``q`` [B,H,Nq,d] against the key/value
    cache ``k``, ``v`` [B,H,Nk,d] (bf16); causal queries are the last Nq
    positions."""
    import torch
    _check(q, "q", dtype=torch.bfloat16)
    _check(k, "k", dtype=torch.bfloat16)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, d):
        raise ValueError(f"k has shape {tuple(k.shape)}, expected {(B, H, Nk, d)}")
    _check(v, "v", k.shape, torch.bfloat16)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), device=q.device, dtype=torch.float32)
    _check(out, "out", q.shape, torch.bfloat16)
    _check(lse, "lse", (B, H, Nq), torch.float32)
    need = fa_decode_workspace_bytes(B, H, Nq, Nk, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    _check(workspace, "workspace")
    rc = fa_decode_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                       workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                       B, H, Nq, Nk, d, float(scale), causal, _stream_ptr(q.device, stream))
    if rc != FA_OK:
        raise FAError(rc, "fa_decode_fwd")
    return out, lse


# ----------------------------------------------------------------- autograd
_AttentionFn = None


def _attention_fn():
    """torch.autograd.Function over fa_fwd / fa_bwd, built on first use (so
    that importing this module does not import torch)."""
    global _AttentionFn
    if _AttentionFn is None:
        import torch

        class AttentionFn(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, causal, scale):
                o, lse = fwd(q, k, v, causal=causal, scale=scale)
                ctx.save_for_backward(q, k, v, o, lse)
                ctx.causal, ctx.scale = causal, scale
                return o

            @staticmethod
            def backward(ctx, grad_o):
                q, k, v, o, lse = ctx.saved_tensors
                do = grad_o
                if do.dtype != torch.bfloat16 or not do.is_contiguous():
                    do = do.to(torch.bfloat16).contiguous()
                dq, dk, dv = bwd(q, k, v, o, do, lse, causal=ctx.causal, scale=ctx.scale)
                return dq, dk, dv, None, None

        _AttentionFn = AttentionFn
    return _AttentionFn


def attention(q, k, v, *, causal: bool = False, scale: float | None = None):
    """O = softmax(scale * Q K^T) V for bf16 [B,H,N,d] GPU tensors, as an
    autograd operation: the forward pass is ``fwd`` (the per-row logsumexp is
    kept for the backward), the backward pass is ``bwd`` on the incoming
    gradient (converted to contiguous bf16 if it is not). Gradients flow to q,
    k and v."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _attention_fn().apply(q, k, v, bool(causal), float(scale))
