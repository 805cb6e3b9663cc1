"""MI355X-native exact attention (FlashAttention-2 order), forward and
backward -- Python binding of the C-ABI library ``libfa2.so`` (declared in ``include/fa2.h``).

This module only marshals arguments: it checks tensor device/dtype/shape,
passes raw device pointers and torch's current HIP stream to the library, and
turns non-zero return codes into exceptions.  Every step of the computation
runs in the library's HIP kernels; there is no fallback.  If the library has
not been built (``python -m exact_io_aware_24_amd.build``) any call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

from . import inputs  # noqa: F401  (seeded synthetic workloads)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa2.so")

# Return codes, mirrored from include/fa2.h.
FA2_OK = 0
FA2_ERR_NULL = -1
FA2_ERR_SHAPE = -2
FA2_ERR_HEADDIM = -3
FA2_ERR_SCALE = -4
FA2_ERR_ALIGN = -5
FA2_ERR_ALIAS = -6
FA2_ERR_HIP = -7
FA2_ERR_WORKSPACE = -8
FA2_ERR_DEVICE = -9
NOALLOC_WORKSPACE_BYTES = 32 << 20  # FA2_NOALLOC_WORKSPACE_BYTES

# Every symbol include/fa2.h declares.
EXPORTED = ("fa2_fwd", "fa2_fwd_o32", "fa2_fwd_gqa", "fa2_fwd_gqa_o32",
            "fa2_fwd_splitkv", "fa2_fwd_splitkv_o32", "fa2_fwd_splitkv_noalloc",
            "fa2_quantize_fp8",
            "fa2_fwd_fp8", "fa2_fwd_fp8_o32", "fa2_fwd_fp32", "fa2_bwd",
            "fa2_bwd_o32", "fa2_bwd_gqa", "fa2_bwd_gqa_o32", "fa2_strerror",
            "fa2_version")
MAX_SPLITS = 1024  # FA2_MAX_SPLITS

_lock = threading.Lock()
_lib = None


class FA2Error(RuntimeError):
    """A non-zero return code from the library."""

    def __init__(self, code: int, func: str):
        self.code = code
        super().__init__("%s failed: %s (code %d)" % (func, strerror(code), code))


def lib() -> ctypes.CDLL:
    """Load ``libfa2.so`` (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libfa2.so is not built: run `python -m exact_io_aware_24_amd.build`"
                " (there is no non-HIP fallback)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i = ctypes.c_void_p, ctypes.c_int
        sig = [vp, vp, vp, vp, vp, i, i, i, i, ctypes.c_float, i, vp]
        for name in ("fa2_fwd", "fa2_fwd_o32", "fa2_fwd_fp32"):
            f = getattr(L, name)
            f.argtypes = sig
            f.restype = ctypes.c_int
        gsig = [vp, vp, vp, vp, vp, i, i, i, i, i, ctypes.c_float, i, vp]
        for name in ("fa2_fwd_gqa", "fa2_fwd_gqa_o32"):
            f = getattr(L, name)
            f.argtypes = gsig
            f.restype = ctypes.c_int
        ssig = [vp] * 5 + [i] * 6 + [ctypes.c_float, i, i, vp, vp, vp]
        for name in ("fa2_fwd_splitkv", "fa2_fwd_splitkv_o32"):
            f = getattr(L, name)
            f.argtypes = ssig
            f.restype = ctypes.c_int
        L.fa2_fwd_splitkv_noalloc.argtypes = [vp] * 5 + [i] * 6 + [ctypes.c_float, i, i, vp]
        L.fa2_fwd_splitkv_noalloc.restype = ctypes.c_int
        L.fa2_quantize_fp8.argtypes = [vp, vp, vp, i, i, i, i, i, vp, vp]
        L.fa2_quantize_fp8.restype = ctypes.c_int
        for name in ("fa2_fwd_fp8", "fa2_fwd_fp8_o32"):
            f = getattr(L, name)
            f.argtypes = [vp] * 8 + [i, i, i, i, ctypes.c_float, i, i, vp]
            f.restype = ctypes.c_int
        bsig = [vp] * 10 + [i, i, i, i, ctypes.c_float, i, vp]
        for name in ("fa2_bwd", "fa2_bwd_o32"):
            f = getattr(L, name)
            f.argtypes = bsig
            f.restype = ctypes.c_int
        gbsig = [vp] * 10 + [i] * 5 + [ctypes.c_float, i, i, vp, vp]
        for name in ("fa2_bwd_gqa", "fa2_bwd_gqa_o32"):
            f = getattr(L, name)
            f.argtypes = gbsig
            f.restype = ctypes.c_int
        L.fa2_strerror.argtypes = [i]
        L.fa2_strerror.restype = ctypes.c_char_p
        L.fa2_version.argtypes = []
        L.fa2_version.restype = ctypes.c_int
        _lib = L
        return L


def strerror(code: int) -> str:
    return lib().fa2_strerror(int(code)).decode()


def version() -> int:
    return int(lib().fa2_version())


def _check_tensors(q, k, v, grouped=False):
    """Device, layout and dtype checks.  ``grouped``: k and v may have fewer
    heads than q, a divisor of q's head count."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
        if t.dim() != 4:
            raise ValueError("%s must be [B, H, N, d], got %s" % (name, tuple(t.shape)))
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    same = q.shape == k.shape == v.shape
    grouped_ok = (grouped and k.shape == v.shape and k.shape[0] == q.shape[0]
                  and k.shape[2:] == q.shape[2:] and k.shape[1] >= 1
                  and q.shape[1] % k.shape[1] == 0)
    if not (same or grouped_ok):
        raise ValueError("q, k, v shapes do not match: %s %s %s"
                         % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v dtypes differ")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must be bfloat16 or float32, got %s" % q.dtype)
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v are on different devices")


def _buffer(t, name, shape, dtype, device, workspace=False):
    """An output or workspace tensor: allocated when ``t`` is None, else
    checked to be a contiguous ``dtype`` GPU tensor on ``device`` of exactly
    ``shape`` (``workspace``: of at least that many elements, any shape).
    The kernels write every element the shape implies, so a smaller buffer
    must never reach them."""
    import torch
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    need = math.prod(shape)
    ok = (isinstance(t, torch.Tensor) and t.is_cuda and t.device == device
          and t.dtype == dtype and t.is_contiguous()
          and (t.numel() >= need if workspace else tuple(t.shape) == tuple(shape)))
    if not ok:
        what = ("at least %d elements" % need) if workspace else "shape %s" % (tuple(shape),)
        raise ValueError("%s must be a contiguous %s tensor on %s with %s"
                         % (name, dtype, device, what))
    return t


def forward(q, k, v, causal: bool = False, scale: float | None = None,
            out_dtype=None, out=None, lse=None, return_lse: bool = True):
    """Exact attention forward: ``softmax(scale * q k^T [+ causal mask]) v``.

    ``q, k, v``: contiguous GPU tensors ``[B, H, N, d]``, d in {64, 128},
    all bfloat16 (MFMA path) or all float32 (fp32 path).  With bfloat16
    inputs ``k`` and ``v`` may be ``[B, H_kv, N, d]`` with H_kv dividing H
    (grouped-query attention, ``fa2_fwd_gqa[_o32]``): query head h uses
    key/value head ``h // (H // H_kv)``.
    ``out_dtype``: for bf16 inputs, ``torch.bfloat16`` (default, entry point
    ``fa2_fwd``) or ``torch.float32`` (``fa2_fwd_o32``); float32 inputs give
    float32 output (``fa2_fwd_fp32``).  ``scale`` defaults to ``1/sqrt(d)``.
    ``out`` / ``lse`` may be preallocated.  Returns ``(o, lse)`` (``lse`` is
    float32 ``[B, H, N]``, or None when ``return_lse`` is False).
    The kernel is enqueued on torch's current stream.
    """
    import torch
    _check_tensors(q, k, v, grouped=True)
    B, H, N, d = (int(x) for x in q.shape)
    H_kv = int(k.shape[1])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if H_kv != H and q.dtype != torch.bfloat16:
        raise ValueError("grouped K/V heads need bfloat16 inputs")
    if q.dtype == torch.float32:
        if out_dtype not in (None, torch.float32):
            raise ValueError("float32 inputs give float32 output")
        fn, odt = "fa2_fwd_fp32", torch.float32
    else:
        odt = torch.bfloat16 if out_dtype is None else out_dtype
        if odt == torch.bfloat16:
            fn = "fa2_fwd"
        elif odt == torch.float32:
            fn = "fa2_fwd_o32"
        else:
            raise ValueError("out_dtype must be bfloat16 or float32")
        if H_kv != H:
            fn = fn.replace("fa2_fwd", "fa2_fwd_gqa")
    out = _buffer(out, "out", (B, H, N, d), odt, q.device)
    lse = _buffer(lse, "lse", (B, H, N), torch.float32, q.device) if return_lse else None
    heads = (B, H, H_kv) if H_kv != H else (B, H)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = getattr(lib(), fn)(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            lse.data_ptr() if lse is not None else None,
            *heads, N, d, ctypes.c_float(scale), int(bool(causal)), stream)
    if rc != FA2_OK:
        raise FA2Error(rc, fn)
    return out, lse


def raw_call(fn: str, q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, N, d, scale,
             causal, stream=None, H_kv=None) -> int:
    """Call a forward entry point with raw integer pointers; returns the
    code.  ``H_kv`` is passed only to the grouped (``_gqa``) entry points."""
    heads = (B, H) if H_kv is None else (B, H, H_kv)
    return int(getattr(lib(), fn)(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, *heads, N,
                                  d, ctypes.c_float(scale), int(causal), stream))


def default_gsplits(B: int, H: int, H_kv: int, N: int) -> int:
    """A count of query-head ranges per shared K/V head for the grouped
    backward that gives the dK/dV kernel about 1024 workgroups (two per
    compute unit, twice over), at most one range per query head."""
    units = B * H_kv * ((N + 127) // 128)
    return int(max(1, min(H // H_kv, -(-1024 // units))))


def backward(q, k, v, o, dout, lse, causal: bool = False,
             scale: float | None = None, out_dtype=None, dq=None, dk=None,
             dv=None, delta=None, n_gsplits: int | None = None, dkv_part=None):
    """Gradients of :func:`forward` with respect to ``q, k, v``.

    ``q, o, dout``: contiguous bfloat16 GPU tensors ``[B, H, N, d]`` (the
    forward's query input and output, and the gradient of the loss with
    respect to ``o``); ``k, v``: ``[B, H, N, d]`` or, with key/value heads
    shared by groups of query heads, ``[B, H_kv, N, d]``; ``lse``: the
    forward's float32 ``[B, H, N]``.  ``causal`` and ``scale`` must be the
    forward's.  ``out_dtype``: ``torch.bfloat16`` (default, ``fa2_bwd``) or
    ``torch.float32`` (``fa2_bwd_o32``); grouped K/V heads call
    ``fa2_bwd_gqa[_o32]`` with ``n_gsplits`` query-head ranges per K/V head
    (default :func:`default_gsplits`) and the float32 workspace
    ``dkv_part`` ``[2, n_gsplits, B, H_kv, N, d]`` (allocated when needed
    and not given).  ``dq, dk, dv`` and the float32 ``[B, H, N]`` workspace
    ``delta`` may be preallocated.  Returns ``(dq, dk, dv)``.  The kernels
    are enqueued on torch's current stream.
    """
    import torch
    _check_tensors(q, k, v, grouped=True)
    _check_tensors(o, dout, q)
    if q.dtype != torch.bfloat16 or o.dtype != torch.bfloat16 \
            or dout.dtype != torch.bfloat16:
        raise ValueError("q, k, v, o and dout must be bfloat16")
    B, H, N, d = (int(x) for x in q.shape)
    Hk = int(k.shape[1])
    grouped = Hk != H or n_gsplits is not None
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    odt = torch.bfloat16 if out_dtype is None else out_dtype
    if odt == torch.bfloat16:
        fn = "fa2_bwd_gqa" if grouped else "fa2_bwd"
    elif odt == torch.float32:
        fn = "fa2_bwd_gqa_o32" if grouped else "fa2_bwd_o32"
    else:
        raise ValueError("out_dtype must be bfloat16 or float32")

    def vec(t, name):
        if t is None:
            return torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        if t.shape != (B, H, N) or t.dtype != torch.float32 \
                or not t.is_contiguous() or t.device != q.device:
            raise ValueError("%s must be a contiguous float32 [B, H, N] tensor" % name)
        return t

    def grad(t, name, like):
        if t is None:
            return torch.empty(like.shape, dtype=odt, device=q.device)
        if t.shape != like.shape or t.dtype != odt or not t.is_contiguous() \
                or t.device != q.device:
            raise ValueError("%s must be a contiguous %s tensor of shape %s"
                             % (name, odt, tuple(like.shape)))
        return t

    if lse is None:
        raise ValueError("lse (from the forward pass) is required")
    lse = vec(lse, "lse")
    delta = vec(delta, "delta")
    dq, dk, dv = grad(dq, "dq", q), grad(dk, "dk", k), grad(dv, "dv", v)
    if grouped:
        ns = default_gsplits(B, H, Hk, N) if n_gsplits is None else int(n_gsplits)
        if not 1 <= ns <= H // Hk:  # before the workspace is sized from it
            raise ValueError("n_gsplits must be in 1..H / H_kv = %d" % (H // Hk))
        if ns > 1 and dkv_part is None:
            dkv_part = torch.empty((2, ns, B, Hk, N, d), dtype=torch.float32,
                                   device=q.device)
        if ns > 1 and (dkv_part.dtype != torch.float32 or not dkv_part.is_contiguous()
                       or dkv_part.numel() < 2 * ns * B * Hk * N * d
                       or dkv_part.device != q.device):
            raise ValueError("dkv_part must be a contiguous float32 tensor of at "
                             "least 2 * n_gsplits * B * H_kv * N * d elements")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                dout.data_ptr(), lse.data_ptr(), delta.data_ptr(), dq.data_ptr(),
                dk.data_ptr(), dv.data_ptr())
        if grouped:
            rc = getattr(lib(), fn)(
                *ptrs, B, H, Hk, N, d, ctypes.c_float(scale), int(bool(causal)),
                ns, dkv_part.data_ptr() if ns > 1 else None, stream)
        else:
            rc = getattr(lib(), fn)(*ptrs, B, H, N, d, ctypes.c_float(scale),
                                    int(bool(causal)), stream)
    if rc != FA2_OK:
        raise FA2Error(rc, fn)
    return dq, dk, dv


def default_splits(B: int, H: int, Nq: int, Nk: int, d: int, H_kv: int | None = None,
                   causal: bool = False) -> int:
    """A key-range count for :func:`forward_splitkv`.  With K/V heads shared
    by H / H_kv query heads, fewer than 128 queries per head and every query
    seeing the same keys (no mask, or one query), the library runs a group's
    rows in one workgroup, and the block count follows that.  Measured on
    decode and chunked-prefill shapes, about 512 workgroups in all (two per
    compute unit) did best.  Blocks with fewer than 128 rows are bound by
    streaming K and V and keep ranges of at least 32 key tiles, except that
    fewer than about 256 workgroups may take ranges down to 16 tiles; full
    blocks keep ranges of at least four tiles."""
    hk = H if H_kv is None else H_kv
    packed = hk < H and Nq < 128 and (Nq == 1 or not causal)
    rows = Nq * (H // hk) if packed else Nq
    blocks = B * (hk if packed else H) * ((rows + 127) // 128)
    tiles = (Nk + 63) // 64  # keys per tile of the bf16 kernels: 64 at both d
    n = -(-512 // blocks)
    if rows < 128:
        floor = min(-(-256 // blocks), tiles // 16)
        n = max(min(n, tiles // 32), floor)
    else:
        n = min(n, tiles // 4)
    return int(max(1, min(n, MAX_SPLITS)))


def forward_splitkv(q, k, v, causal: bool = False, scale: float | None = None,
                    n_splits: int | None = None, out_dtype=None, out=None,
                    lse=None, o_part=None, lse_part=None, return_lse: bool = True):
    """General forward (``fa2_fwd_splitkv[_o32]``): ``q`` ``[B, H, Nq, d]``
    against ``k, v`` ``[B, H_kv, Nk, d]`` (bfloat16, H_kv dividing H), the
    keys of each query block split into ``n_splits`` ranges that are merged
    afterwards (default: :func:`default_splits`).  Causal: query i sits at
    key position ``i + Nk - Nq``.  Workspaces ``o_part`` (float32
    ``[n_splits, B, H, Nq, d]``) and ``lse_part`` (``[n_splits, B, H, Nq]``)
    are allocated when not given.  Returns ``(o, lse)``."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4 or not t.is_cuda \
                or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError("%s must be a contiguous bfloat16 GPU tensor [B, H, N, d]" % name)
    B, H, Nq, d = (int(x) for x in q.shape)
    H_kv, Nk = int(k.shape[1]), int(k.shape[2])
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d or H_kv < 1 \
            or H % H_kv != 0 or not (q.device == k.device == v.device):
        raise ValueError("k, v must be [B, H_kv, Nk, d] with H_kv dividing H")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if n_splits is None:
        n_splits = default_splits(B, H, Nq, Nk, d, H_kv, causal)
    if not 1 <= int(n_splits) <= MAX_SPLITS:  # before any workspace is sized from it
        raise ValueError("n_splits must be in 1..%d" % MAX_SPLITS)
    odt = torch.bfloat16 if out_dtype is None else out_dtype
    fn = {torch.bfloat16: "fa2_fwd_splitkv", torch.float32: "fa2_fwd_splitkv_o32"}.get(odt)
    if fn is None:
        raise ValueError("out_dtype must be bfloat16 or float32")
    dev = q.device
    out = _buffer(out, "out", (B, H, Nq, d), odt, dev)
    lse = _buffer(lse, "lse", (B, H, Nq), torch.float32, dev) if return_lse else None
    if n_splits > 1:
        o_part = _buffer(o_part, "o_part", (n_splits, B, H, Nq, d), torch.float32, dev,
                         workspace=True)
        lse_part = _buffer(lse_part, "lse_part", (n_splits, B, H, Nq), torch.float32, dev,
                           workspace=True)
    ptr = lambda t: t.data_ptr() if t is not None else None
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = getattr(lib(), fn)(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), ptr(lse),
            B, H, H_kv, Nq, Nk, d, ctypes.c_float(scale), int(bool(causal)),
            int(n_splits), ptr(o_part), ptr(lse_part), stream)
    if rc != FA2_OK:
        raise FA2Error(rc, fn)
    return out, lse


def forward_splitkv_noalloc(q, k, v, causal: bool = False,
                            scale: float | None = None, n_splits: int | None = None,
                            out=None, lse=None, return_lse: bool = True):
    """``fa2_fwd_splitkv_noalloc``: :func:`forward_splitkv` (bf16 output)
    with the key-range partials in the library's static device workspace.
    ``out`` and ``lse`` are allocated here when not given (torch memory);
    pass them to keep the call allocation-free.  Returns ``(o, lse)``."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4 or not t.is_cuda \
                or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError("%s must be a contiguous bfloat16 GPU tensor [B, H, N, d]" % name)
    B, H, Nq, d = (int(x) for x in q.shape)
    H_kv, Nk = int(k.shape[1]), int(k.shape[2])
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d or H_kv < 1 \
            or H % H_kv != 0 or not (q.device == k.device == v.device):
        raise ValueError("k, v must be [B, H_kv, Nk, d] with H_kv dividing H")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if n_splits is None:
        n_splits = default_splits(B, H, Nq, Nk, d, H_kv, causal)
    if not 1 <= int(n_splits) <= MAX_SPLITS:
        raise ValueError("n_splits must be in 1..%d" % MAX_SPLITS)
    dev = q.device
    out = _buffer(out, "out", (B, H, Nq, d), torch.bfloat16, dev)
    lse = _buffer(lse, "lse", (B, H, Nq), torch.float32, dev) if return_lse else None
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib().fa2_fwd_splitkv_noalloc(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            lse.data_ptr() if lse is not None else None, B, H, H_kv, Nq, Nk, d,
            ctypes.c_float(scale), int(bool(causal)), int(n_splits), stream)
    if rc != FA2_OK:
        raise FA2Error(rc, "fa2_fwd_splitkv_noalloc")
    return out, lse


def raw_call_splitkv(fn: str, ptrs, B, H, H_kv, Nq, Nk, d, scale, causal,
                     n_splits, stream=None) -> int:
    """Call a split-KV entry point with raw pointers (q, k, v, o, lse,
    o_part, lse_part); returns the code."""
    q, k, v, o, lse, op, lp = ptrs
    return int(getattr(lib(), fn)(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d,
                                  ctypes.c_float(scale), int(causal), n_splits,
                                  op, lp, stream))


def quantize_fp8(x, block_rows: int, signs=None, codes=None, exps=None):
    """Block-quantise a contiguous bfloat16 GPU tensor ``[B, H, N, d]`` to
    e4m3 codes (``fa2_quantize_fp8``), optionally rotating each row by the
    random-sign Walsh-Hadamard transform given by ``signs`` (a float32 GPU
    tensor of d values +-1).  Returns ``(codes uint8 [B, H, N, d], exps int32
    [B, H, ceil(N / block_rows)])``."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dim() != 4 or not x.is_cuda \
            or not x.is_contiguous() or x.dtype != torch.bfloat16:
        raise ValueError("x must be a contiguous bfloat16 GPU tensor [B, H, N, d]")
    B, H, N, d = (int(v) for v in x.shape)
    if block_rows not in (64, 128):
        raise ValueError("block_rows must be 64 or 128")
    nb = -(-N // block_rows)
    codes = _buffer(codes, "codes", (B, H, N, d), torch.uint8, x.device)
    exps = _buffer(exps, "exps", (B, H, nb), torch.int32, x.device)
    if signs is not None and (not isinstance(signs, torch.Tensor)
                              or signs.dtype != torch.float32 or signs.numel() != d
                              or not signs.is_cuda or signs.device != x.device
                              or not signs.is_contiguous()):
        raise ValueError("signs must be a contiguous float32 tensor of d values on "
                         "the device of x")
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        rc = lib().fa2_quantize_fp8(x.data_ptr(), codes.data_ptr(), exps.data_ptr(),
                                    B, H, N, d, int(block_rows),
                                    signs.data_ptr() if signs is not None else None,
                                    stream)
    if rc != FA2_OK:
        raise FA2Error(rc, "fa2_quantize_fp8")
    return codes, exps


def forward_fp8(q8, q_exp, k8, k_exp, v8, v_exp, causal: bool = False,
                scale: float | None = None, rotated: bool = False,
                out_dtype=None, out=None, lse=None):
    """FP8 attention (``fa2_fwd_fp8[_o32]``) of quantised inputs from
    :func:`quantize_fp8` (Q with 128-row blocks, K and V with 64-row blocks,
    Q and K rotated with the same signs iff ``rotated``).  ``scale`` is the
    attention scale of the original inputs (default 1/sqrt(d)).  Returns
    ``(o, lse)``."""
    import torch
    if not isinstance(q8, torch.Tensor) or q8.dim() != 4:
        raise ValueError("q8 must be a uint8 tensor [B, H, N, d]")
    B, H, N, d = (int(v) for v in q8.shape)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    odt = torch.bfloat16 if out_dtype is None else out_dtype
    fn = {torch.bfloat16: "fa2_fwd_fp8", torch.float32: "fa2_fwd_fp8_o32"}.get(odt)
    if fn is None:
        raise ValueError("out_dtype must be bfloat16 or float32")
    dev = q8.device
    for t in (q8, k8, v8):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 \
                or tuple(t.shape) != (B, H, N, d) or not t.is_cuda \
                or t.device != dev or not t.is_contiguous():
            raise ValueError("codes must be contiguous uint8 tensors [B, H, N, d] on one GPU")
    # block exponents: Q per 128-row block, K and V per 64-row block
    for t, name, rows in ((q_exp, "q_exp", 128), (k_exp, "k_exp", 64), (v_exp, "v_exp", 64)):
        shape = (B, H, -(-N // rows))
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 \
                or tuple(t.shape) != shape or not t.is_cuda or t.device != dev \
                or not t.is_contiguous():
            raise ValueError("%s must be a contiguous int32 tensor %s on the device "
                             "of the codes" % (name, shape))
    out = _buffer(out, "out", (B, H, N, d), odt, dev)
    lse = _buffer(lse, "lse", (B, H, N), torch.float32, dev)
    with torch.cuda.device(q8.device):
        stream = torch.cuda.current_stream(q8.device).cuda_stream
        rc = getattr(lib(), fn)(q8.data_ptr(), q_exp.data_ptr(), k8.data_ptr(),
                                k_exp.data_ptr(), v8.data_ptr(), v_exp.data_ptr(),
                                out.data_ptr(), lse.data_ptr(), B, H, N, d,
                                ctypes.c_float(scale), int(bool(rotated)),
                                int(bool(causal)), stream)
    if rc != FA2_OK:
        raise FA2Error(rc, fn)
    return out, lse


def attention_fp8(q, k, v, causal: bool = False, scale: float | None = None,
                  signs=None, out_dtype=None):
    """bf16 ``q, k, v`` -> FP8 attention: quantise (Q and K rotated by
    ``signs`` when given), then :func:`forward_fp8`.  Returns ``(o, lse)``."""
    q8, qe = quantize_fp8(q, 128, signs)
    k8, ke = quantize_fp8(k, 64, signs)
    v8, ve = quantize_fp8(v, 64, None)
    return forward_fp8(q8, qe, k8, ke, v8, ve, causal=causal, scale=scale,
                       rotated=signs is not None, out_dtype=out_dtype)


def raw_call_bwd(fn: str, ptrs, B, H, N, d, scale, causal, stream=None) -> int:
    """Call a backward entry point with ten raw integer pointers (q, k, v, o,
    dout, lse, delta, dq, dk, dv); returns the code."""
    if len(ptrs) != 10:
        raise ValueError("ten pointers expected")
    return int(getattr(lib(), fn)(*ptrs, B, H, N, d, ctypes.c_float(scale),
                                  int(causal), stream))


def raw_call_bwd_gqa(fn: str, ptrs, B, H, H_kv, N, d, scale, causal, n_gsplits,
                     dkv_part, stream=None) -> int:
    """Call a grouped backward entry point with ten raw integer pointers (as
    :func:`raw_call_bwd`) and the raw workspace pointer; returns the code."""
    if len(ptrs) != 10:
        raise ValueError("ten pointers expected")
    return int(getattr(lib(), fn)(*ptrs, B, H, H_kv, N, d, ctypes.c_float(scale),
                                  int(causal), n_gsplits, dkv_part, stream))


_ATTENTION_FN = None


def _attention_fn():
    """The autograd Function behind :func:`attention` (built on first use so
    that importing the package does not import torch)."""
    global _ATTENTION_FN
    if _ATTENTION_FN is None:
        import torch

        class _Attention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, causal, scale):
                o, lse = forward(q, k, v, causal=causal, scale=scale)
                ctx.save_for_backward(q, k, v, o, lse)
                ctx.causal, ctx.scale = causal, scale
                return o

            @staticmethod
            def backward(ctx, do):
                q, k, v, o, lse = ctx.saved_tensors
                dq, dk, dv = backward(q, k, v, o, do.contiguous(), lse,
                                      causal=ctx.causal, scale=ctx.scale)
                return dq, dk, dv, None, None

        _ATTENTION_FN = _Attention
    return _ATTENTION_FN


def attention(q, k, v, causal: bool = False, scale: float | None = None):
    """Exact attention as a differentiable torch operation: the output of
    :func:`forward` (bfloat16 ``[B, H, N, d]``), whose gradient with respect
    to ``q, k, v`` :func:`backward` computes from the saved output and
    log-sum-exp.  ``q``: ``[B, H, N, d]``, ``k, v``: ``[B, H, N, d]`` or
    ``[B, H_kv, N, d]`` with H_kv dividing H; all contiguous bfloat16 GPU
    tensors (the backward pass exists for bfloat16 only).  Both passes are
    enqueued on torch's current stream."""
    import torch
    _check_tensors(q, k, v, grouped=True)
    if q.dtype != torch.bfloat16:
        raise ValueError("attention() needs bfloat16 q, k, v (the backward pass is bf16)")
    d = int(q.shape[-1])
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    return _attention_fn().apply(q, k, v, bool(causal), s)
