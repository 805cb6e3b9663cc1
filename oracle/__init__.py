"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never links, loads or
calls it, and it shares no code with the GPU path.

The arithmetic lives in ``attn_oracle.c`` (plain C, IEEE double precision,
POSIX threads over independent query rows); this module only builds it with
gcc and marshals numpy arrays into it.  What is computed, and the page passage
each step follows, is stated in the C file's header:

* ``S = scale * Q K^T`` row by row, causal keys ``j > i`` at ``-inf``;
* ``P = softmax(S)`` with the row maximum subtracted first;
* ``O = P V`` and ``lse = m + ln(sum exp(S - m))`` (natural log);
* the exact gradients ``dQ, dK, dV`` of that definition for an incoming
  gradient ``dO`` (``dV = P^T dO``, ``dS = P * (dO V^T - D)``,
  ``dQ = scale dS K``, ``dK = scale dS^T Q``, ``D_i = sum_j P_ij dP_ij``);
* FP8 block quantisation with incoherent processing (``quantize_fp8``):
  a random-sign Walsh-Hadamard rotation, a power-of-two scale per block of
  rows, e4m3 codes -- the FlashAttention-3 FP8 recipe of the itimpress.au
  page, section 1.

Every function here is pinned by ``tests/test_oracle_pins.py`` (closed forms,
invariants, the two-block merge rule from the online-softmax section of the
"Large language models part 06" page, and brute force on tiny shapes).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle's C source into a shared library with gcc.

    -O2 without fast-math and with ``-ffp-contract=off``: the compiler may not
    reassociate or fuse the double-precision arithmetic, so the oracle is the
    written definition evaluated in IEEE order.  ``src``/``out`` exist so the
    tests can also build deliberately broken copies of the oracle and check
    that its pins catch them.
    """
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-pthread", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _f64(a) -> np.ndarray:
    """Any array-like (numpy, or a CPU torch tensor of any float dtype) to a
    C-contiguous float64 numpy array holding exactly the same values."""
    if hasattr(a, "detach"):  # torch tensor: widen on the torch side first,
        a = a.detach().cpu()  # numpy has no bfloat16
        import torch
        a = a.to(torch.float64).numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


class OracleLib:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.oracle_attention_f64.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64,
                                             i64, ctypes.c_double, ctypes.c_int,
                                             ctypes.c_int]
        lib.oracle_attention_f64.restype = ctypes.c_int
        lib.oracle_attention_rows_f64.argtypes = [
            dp, ctypes.POINTER(i64), i64, dp, dp, i64, i64, ctypes.c_double,
            ctypes.c_int, dp, dp, ctypes.c_int]
        lib.oracle_attention_rows_f64.restype = ctypes.c_int
        lib.oracle_probs_f64.argtypes = [dp, dp, i64, i64, i64, ctypes.c_double,
                                         ctypes.c_int, dp, dp, dp]
        lib.oracle_probs_f64.restype = ctypes.c_int
        lib.oracle_attention_bwd_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp,
                                                 dp, i64, i64, i64, i64,
                                                 ctypes.c_double, ctypes.c_int,
                                                 ctypes.c_int]
        lib.oracle_attention_bwd_f64.restype = ctypes.c_int
        lib.oracle_default_threads.argtypes = []
        lib.oracle_default_threads.restype = ctypes.c_int
        self.path = path
        self._lib = lib

    def default_threads(self) -> int:
        """Host cores this process may run on (``sched_getaffinity``)."""
        return int(self._lib.oracle_default_threads())

    def attention(self, q, k, v, scale: float, causal: bool = False,
                  nthreads: int = 0):
        """Exact attention of every head.

        ``q``: ``[..., Nq, d]``; ``k``, ``v``: ``[..., Nk, d]`` with the same
        leading (head) dimensions.  Returns ``(o, lse, threads_used)`` with
        ``o`` ``[..., Nq, d]`` and ``lse`` ``[..., Nq]``, both float64.
        """
        q, k, v = _f64(q), _f64(k), _f64(v)
        if q.ndim < 2 or k.shape != v.shape or q.shape[:-2] != k.shape[:-2] \
                or q.shape[-1] != k.shape[-1]:
            raise ValueError("shape mismatch: q %s k %s v %s"
                             % (q.shape, k.shape, v.shape))
        lead = q.shape[:-2]
        nq, d = q.shape[-2], q.shape[-1]
        nk = k.shape[-2]
        nh = int(np.prod(lead)) if lead else 1
        o = np.empty(q.shape, dtype=np.float64)
        lse = np.empty(lead + (nq,), dtype=np.float64)
        rc = self._lib.oracle_attention_f64(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), nh, nq, nk, d,
            float(scale), int(bool(causal)), int(nthreads))
        if rc < 0:
            raise RuntimeError("oracle_attention_f64 failed (%d)" % rc)
        return o, lse, rc

    def attention_rows(self, q_rows, rows, k, v, scale: float,
                       causal: bool = False, nthreads: int = 0):
        """Exact attention of selected query rows of ONE head.

        ``q_rows``: ``[R, d]`` query vectors, ``rows``: ``[R]`` their row
        indices (the causal mask needs them), ``k``, ``v``: ``[Nk, d]``.
        Returns ``(o [R, d], lse [R], threads_used)``.
        """
        q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        if q_rows.ndim != 2 or rows.shape != (q_rows.shape[0],) or k.ndim != 2 \
                or k.shape != v.shape or k.shape[1] != q_rows.shape[1]:
            raise ValueError("shape mismatch")
        nr, d = q_rows.shape
        o = np.empty((nr, d), dtype=np.float64)
        lse = np.empty((nr,), dtype=np.float64)
        rc = self._lib.oracle_attention_rows_f64(
            _ptr(q_rows), rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
            nr, _ptr(k), _ptr(v), k.shape[0], d, float(scale),
            int(bool(causal)), _ptr(o), _ptr(lse), int(nthreads))
        if rc < 0:
            raise RuntimeError("oracle_attention_rows_f64 failed (%d)" % rc)
        return o, lse, rc

    def attention_bwd(self, q, k, v, dout, scale: float, causal: bool = False,
                      nthreads: int = 0):
        """Exact gradients of every head for the incoming gradient ``dout``
        of the output.

        ``q``, ``dout``: ``[..., Nq, d]``; ``k``, ``v``: ``[..., Nk, d]``.
        Returns ``(dq, dk, dv, delta, threads_used)`` (float64) where
        ``delta[..., i] = sum_j P_ij dP_ij``.
        """
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        if q.ndim < 2 or k.shape != v.shape or q.shape != dout.shape or \
                q.shape[:-2] != k.shape[:-2] or q.shape[-1] != k.shape[-1]:
            raise ValueError("shape mismatch: q %s k %s v %s dout %s"
                             % (q.shape, k.shape, v.shape, dout.shape))
        lead = q.shape[:-2]
        nq, d = q.shape[-2], q.shape[-1]
        nk = k.shape[-2]
        nh = int(np.prod(lead)) if lead else 1
        dq = np.empty(q.shape, dtype=np.float64)
        dk = np.empty(k.shape, dtype=np.float64)
        dv = np.empty(v.shape, dtype=np.float64)
        delta = np.empty(lead + (nq,), dtype=np.float64)
        rc = self._lib.oracle_attention_bwd_f64(
            _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(delta), nh, nq, nk, d, float(scale), int(bool(causal)),
            int(nthreads))
        if rc < 0:
            raise RuntimeError("oracle_attention_bwd_f64 failed (%d)" % rc)
        return dq, dk, dv, delta, rc

    def probs(self, q, k, scale: float, causal: bool = False):
        """The probability matrix of ONE head: ``(P [Nq, Nk], m [Nq], l [Nq])``
        where ``m`` is each row's maximum score and ``l = sum_j exp(s_j - m)``.
        """
        q, k = _f64(q), _f64(k)
        if q.ndim != 2 or k.ndim != 2 or q.shape[1] != k.shape[1]:
            raise ValueError("shape mismatch")
        nq, nk, d = q.shape[0], k.shape[0], q.shape[1]
        p = np.empty((nq, nk), dtype=np.float64)
        m = np.empty((nq,), dtype=np.float64)
        l = np.empty((nq,), dtype=np.float64)
        rc = self._lib.oracle_probs_f64(_ptr(q), _ptr(k), nq, nk, d,
                                        float(scale), int(bool(causal)),
                                        _ptr(p), _ptr(m), _ptr(l))
        if rc < 0:
            raise RuntimeError("oracle_probs_f64 failed (%d)" % rc)
        return p, m, l


def _default() -> OracleLib:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or (
                    os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
                build(force=True)
            _lib = OracleLib(_LIB_PATH)
        return _lib


def default_threads() -> int:
    return _default().default_threads()


def attention(q, k, v, scale: float, causal: bool = False, nthreads: int = 0):
    return _default().attention(q, k, v, scale, causal, nthreads)


def attention_rows(q_rows, rows, k, v, scale: float, causal: bool = False,
                   nthreads: int = 0):
    return _default().attention_rows(q_rows, rows, k, v, scale, causal,
                                     nthreads)


def probs(q, k, scale: float, causal: bool = False):
    return _default().probs(q, k, scale, causal)


def attention_bwd(q, k, v, dout, scale: float, causal: bool = False,
                  nthreads: int = 0):
    return _default().attention_bwd(q, k, v, dout, scale, causal, nthreads)


def expand_kv_heads(kv, heads: int):
    """Grouped-query attention by its definition: query head h of H uses
    key/value head h // (H / H_kv).  ``kv``: ``[..., H_kv, N, d]``; returns
    ``[..., H, N, d]`` float64 with each K/V head repeated for its group of
    consecutive query heads."""
    kv = _f64(kv)
    hk = kv.shape[-3]
    if heads % hk != 0:
        raise ValueError("H_kv = %d does not divide H = %d" % (hk, heads))
    return np.repeat(kv, heads // hk, axis=-3)


def attention_offset(q, k, v, scale: float, causal: bool = False,
                     nthreads: int = 0):
    """Exact attention of ``q`` ``[..., Nq, d]`` against ``k, v``
    ``[..., Nk, d]`` (same heads) with the causal mask aligned at the end of
    the keys: query i is at key position ``i + Nk - Nq`` and sees the keys at
    or before it -- the rows ``Nk - Nq .. Nk - 1`` of the square problem
    over all Nk positions.  Rows with no visible key get O = 0, lse = -inf.
    Returns ``(o, lse, threads_used)``."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    nq, nk, d = q.shape[-2], k.shape[-2], q.shape[-1]
    if not causal or nq == nk:
        return attention(q, k, v, scale, causal, nthreads)
    lead = q.shape[:-2]
    qh = q.reshape(-1, nq, d)
    kh, vh = k.reshape(-1, nk, d), v.reshape(-1, nk, d)
    rows = np.arange(nq, dtype=np.int64) + (nk - nq)
    o = np.empty(qh.shape)
    lse = np.empty(qh.shape[:2])
    used = 0
    for h in range(qh.shape[0]):
        o[h], lse[h], used = attention_rows(qh[h], rows, kh[h], vh[h], scale,
                                            True, nthreads)
    return o.reshape(lead + (nq, d)), lse.reshape(lead + (nq,)), used


def attention_gqa(q, k, v, scale: float, causal: bool = False, nthreads: int = 0):
    """Exact attention with grouped K/V heads: ``q`` ``[..., H, N, d]``,
    ``k``, ``v`` ``[..., H_kv, N, d]`` (H_kv dividing H).  Returns
    ``(o, lse, threads_used)`` as :func:`attention`."""
    h = _f64(q).shape[-3]
    return attention(q, expand_kv_heads(k, h), expand_kv_heads(v, h), scale,
                     causal, nthreads)


def sum_kv_groups(x, heads_kv: int):
    """Inverse of :func:`expand_kv_heads` for gradients: ``x`` ``[..., H, N,
    d]`` summed over each group of H / H_kv consecutive query heads into
    ``[..., H_kv, N, d]`` (a K/V head used by several query heads receives
    the sum of their gradients)."""
    x = _f64(x)
    h = x.shape[-3]
    if h % heads_kv != 0:
        raise ValueError("H_kv = %d does not divide H = %d" % (heads_kv, h))
    shape = x.shape[:-3] + (heads_kv, h // heads_kv) + x.shape[-2:]
    return x.reshape(shape).sum(axis=-3)


def attention_bwd_gqa(q, k, v, dout, scale: float, causal: bool = False,
                      nthreads: int = 0):
    """Gradients of the grouped-head attention (:func:`attention_gqa`):
    the plain backward on the expanded K/V, then dK, dV summed over each
    group.  Returns ``(dq, dk, dv, delta, threads_used)`` with dk, dv of
    shape ``[..., H_kv, N, d]``."""
    h = _f64(q).shape[-3]
    hk = _f64(k).shape[-3]
    dq, dk, dv, delta, used = attention_bwd(q, expand_kv_heads(k, h),
                                            expand_kv_heads(v, h), dout, scale,
                                            causal, nthreads)
    return dq, sum_kv_groups(dk, hk), sum_kv_groups(dv, hk), delta, used

# ---------------------------------------------------------------------------
# FP8 block quantisation (itimpress.au page "FlashAttention scaling, multi-GPU
# training and weight quantisation", section 1: small tiles scaled
# independently; Q and K multiplied by a random orthogonal matrix first).

E4M3_MAX = 448.0


def fwht_f32(x):
    """Unnormalised Walsh-Hadamard transform of the last axis (a power of
    two), in float32, one butterfly stage at a time for h = 1, 2, 4, ...:
    (a, b) -> (a + b, a - b) for every pair (i, i + h) inside blocks of 2h.
    Each output of a stage is one IEEE float32 addition, so any
    implementation with the same stages gives the same bits.  Applying it
    twice multiplies by the length."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("length must be a power of two")
    h = 1
    while h < d:
        z = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = z[..., 0, :].copy()
        b = z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(y.shape)
        h *= 2
    return y


def block_exponent(amax):
    """Smallest integer e with amax <= 448 * 2^e (0 for amax == 0): the
    power-of-two scale that maps a block's largest magnitude into the e4m3
    range."""
    # amax = m * 2^E with 0.5 <= m < 1 and 448 = 0.875 * 2^9, so
    # amax <= 448 * 2^e  <=>  m * 2^E <= 0.875 * 2^(9 + e): the smallest such
    # e is E - 9 when m <= 0.875 and E - 8 otherwise (no rounded division)
    amax = np.asarray(amax, dtype=np.float64)
    m, ex = np.frexp(amax)
    e = np.where(m <= 0.875, ex - 9, ex - 8).astype(np.int32)
    return np.where(amax > 0, e, 0).astype(np.int32)


def to_e4m3_codes(x):
    """Round float32 values to e4m3 (OCP FP8, round to nearest even) and
    return the codes as uint8 (torch's float8_e4m3fn conversion)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_values(codes):
    """The float64 values of e4m3 codes."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def quantize_fp8(x, block_rows: int, signs=None):
    """Block-quantise ``x`` ``[..., N, d]`` (exact values, e.g. bf16).

    With ``signs`` (``d`` values of +-1) each row is first multiplied by the
    signs and transformed with :func:`fwht_f32` -- the rotation by the
    orthogonal matrix diag(signs) H / sqrt(d), with the 1/sqrt(d) left to
    the caller.  Each block of ``block_rows`` rows (per leading index) gets
    the exponent e of :func:`block_exponent` for its largest magnitude and
    stores e4m3(y * 2^-e).  Returns ``(codes uint8 [..., N, d], exps int32
    [..., ceil(N / block_rows)])``; the dequantised value is
    ``e4m3_values(codes) * 2^e``."""
    y = np.asarray(_f64(x), dtype=np.float32)  # exact for bf16 inputs
    if signs is not None:
        y = fwht_f32(y * np.asarray(signs, dtype=np.float32))
    n, d = y.shape[-2], y.shape[-1]
    nb = -(-n // block_rows)
    pad = nb * block_rows - n
    yp = np.concatenate([y, np.zeros(y.shape[:-2] + (pad, d), np.float32)], axis=-2) if pad else y
    blocks = yp.reshape(yp.shape[:-2] + (nb, block_rows, d))
    amax = np.abs(blocks).max(axis=(-2, -1))
    e = block_exponent(amax)
    scaled = blocks * np.ldexp(np.float32(1), -e)[..., None, None].astype(np.float32)
    codes = to_e4m3_codes(scaled).reshape(yp.shape)
    return codes[..., :n, :], e


def dequantize_fp8(codes, exps, block_rows: int):
    """float64 values of block-quantised codes (see :func:`quantize_fp8`)."""
    v = e4m3_values(codes)
    n = v.shape[-2]
    rep = np.repeat(exps, block_rows, axis=-1)[..., :n].astype(np.float64)
    return v * np.exp2(rep)[..., None]


def attention_fp8_reference(q, k, v, scale: float, causal: bool = False,
                            signs=None, q_rows: int = 128, kv_rows: int = 64):
    """Exact attention (fp64) of the block-quantised inputs: what an FP8
    kernel computes before its own roundings (of P and of the output).
    Q and K are quantised with ``signs`` (rotation) if given, Q in blocks of
    ``q_rows`` rows, K and V in blocks of ``kv_rows``; the rotation's
    1/sqrt(d) factors multiply into scale / d.  Returns ``(o, lse, codes)``
    with ``codes = ((q8, qe), (k8, ke), (v8, ve))``."""
    d = _f64(q).shape[-1]
    q8, qe = quantize_fp8(q, q_rows, signs)
    k8, ke = quantize_fp8(k, kv_rows, signs)
    v8, ve = quantize_fp8(v, kv_rows, None)
    qd = dequantize_fp8(q8, qe, q_rows)
    kd = dequantize_fp8(k8, ke, kv_rows)
    vd = dequantize_fp8(v8, ve, kv_rows)
    s_eff = scale / d if signs is not None else scale
    o, lse, _ = attention(qd, kd, vd, s_eff, causal)
    return o, lse, ((q8, qe), (k8, ke), (v8, ve))