"""Host-side checks of the C-ABI library that need no GPU: it loads, it
exports every symbol include/fa2.h declares, and every argument error is
reported before any HIP call (so these calls never touch a device)."""
import ctypes
import os
import re
import subprocess

import pytest

import exact_io_aware_24_amd as fa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")


def header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(fa2_\w+)\s*\(", txt)))


def header_codes():
    return {m.group(1): int(m.group(2)) for m in re.finditer(
        r"#define\s+(FA2_(?:OK|ERR_\w+))\s+\(?(-?\d+)\)?", open(HEADER).read())}


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fa2.LIB_PATH):
        pytest.fail("libfa2.so not built (python -m exact_io_aware_24_amd.build)")
    return fa2.lib()


def test_exports_match_header(L):
    declared = header_functions()
    assert declared == sorted(fa2.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", fa2.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = sorted(set(re.findall(r"\bT\s+(fa2_\w+)$", out, flags=re.M)))
    assert exported == declared
    for name in declared:
        assert getattr(L, name) is not None


def test_codes_match_header():
    codes = header_codes()
    for name, val in codes.items():
        assert getattr(fa2, name) == val, name


def test_version_and_strerror(L):
    assert fa2.version() == 8
    seen = set()
    for name, code in header_codes().items():
        msg = fa2.strerror(code)
        assert msg and msg not in seen
        seen.add(msg)
    assert "unknown" in fa2.strerror(12345)


# Fake, never-dereferenced device addresses: every call below is rejected by
# validation before the library makes any HIP call.
MiB = 1 << 20
Q, K, V, O, LSE = (0x10000000 + i * 64 * MiB for i in range(5))
FUNCS = ("fa2_fwd", "fa2_fwd_o32", "fa2_fwd_fp32")
GOOD = dict(q=Q, k=K, v=V, o=O, lse=LSE, B=1, H=2, N=64, d=64, scale=0.125,
            causal=0)


def call(fn, **kw):
    a = dict(GOOD)
    a.update(kw)
    return fa2.raw_call(fn, a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                        a["H"], a["N"], a["d"], a["scale"], a["causal"])


@pytest.mark.parametrize("fn", FUNCS)
def test_null_pointers(L, fn):
    for key in ("q", "k", "v", "o"):
        assert call(fn, **{key: None}) == fa2.FA2_ERR_NULL


@pytest.mark.parametrize("fn", FUNCS)
def test_bad_shapes(L, fn):
    for kw in (dict(B=0), dict(H=0), dict(N=0), dict(B=-1), dict(N=-5),
               dict(N=1 << 30, d=128),              # N*d over 2^31-1
               dict(B=1 << 16, H=1 << 16, N=1)):     # B*H over 2^31-1
        assert call(fn, **kw) == fa2.FA2_ERR_SHAPE, kw


@pytest.mark.parametrize("fn", FUNCS)
def test_bad_head_dim(L, fn):
    for d in (0, 1, 32, 63, 96, 127, 256):
        assert call(fn, d=d) == fa2.FA2_ERR_HEADDIM, d


@pytest.mark.parametrize("fn", FUNCS)
def test_bad_scale(L, fn):
    for s in (float("nan"), float("inf"), float("-inf")):
        assert call(fn, scale=s) == fa2.FA2_ERR_SCALE


@pytest.mark.parametrize("fn", FUNCS)
def test_misaligned(L, fn):
    for key in ("q", "k", "v", "o", "lse"):
        assert call(fn, **{key: GOOD[key] + 8}) == fa2.FA2_ERR_ALIGN, key


@pytest.mark.parametrize("fn", FUNCS)
def test_aliasing(L, fn):
    assert call(fn, o=Q) == fa2.FA2_ERR_ALIAS
    assert call(fn, o=V + 4096) == fa2.FA2_ERR_ALIAS
    assert call(fn, lse=K) == fa2.FA2_ERR_ALIAS
    assert call(fn, lse=O + 16) == fa2.FA2_ERR_ALIAS


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fa2.forward(q, q, q)


def test_binding_rejects_bad_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa2.forward(q[0], q[0], q[0])
    with pytest.raises(TypeError):
        fa2.forward(None, q, q)


# Backward entry points: ten pointers (q, k, v, o, dout, lse, delta, dq, dk,
# dv), all required.  Again only calls that validation rejects.
BWD_FUNCS = ("fa2_bwd", "fa2_bwd_o32")
BWD_NAMES = ("q", "k", "v", "o", "dout", "lse", "delta", "dq", "dk", "dv")
BWD_GOOD = {name: 0x10000000 + i * 64 * MiB for i, name in enumerate(BWD_NAMES)}
BWD_SHAPE = dict(B=1, H=2, N=64, d=64, scale=0.125, causal=1)


def call_bwd(fn, ptrs=None, **kw):
    p = dict(BWD_GOOD)
    p.update(ptrs or {})
    a = dict(BWD_SHAPE)
    a.update(kw)
    return fa2.raw_call_bwd(fn, [p[n] for n in BWD_NAMES], a["B"], a["H"],
                            a["N"], a["d"], a["scale"], a["causal"])


@pytest.mark.parametrize("fn", BWD_FUNCS)
def test_bwd_null_pointers(L, fn):
    for name in BWD_NAMES:
        assert call_bwd(fn, {name: None}) == fa2.FA2_ERR_NULL, name


@pytest.mark.parametrize("fn", BWD_FUNCS)
def test_bwd_bad_arguments(L, fn):
    for kw in (dict(B=0), dict(H=0), dict(N=0), dict(N=1 << 30, d=128),
               dict(B=1 << 16, H=1 << 16, N=1)):
        assert call_bwd(fn, **kw) == fa2.FA2_ERR_SHAPE, kw
    for d in (0, 32, 96, 256):
        assert call_bwd(fn, d=d) == fa2.FA2_ERR_HEADDIM, d
    for s in (float("nan"), float("inf")):
        assert call_bwd(fn, scale=s) == fa2.FA2_ERR_SCALE
    for name in BWD_NAMES:
        assert call_bwd(fn, {name: BWD_GOOD[name] + 4}) == fa2.FA2_ERR_ALIGN, name


@pytest.mark.parametrize("fn", BWD_FUNCS)
def test_bwd_aliasing(L, fn):
    # every output against every input, and the outputs against each other
    outs = ("delta", "dq", "dk", "dv")
    for o in outs:
        for i in ("q", "k", "v", "o", "dout", "lse"):
            assert call_bwd(fn, {o: BWD_GOOD[i] + 16}) == fa2.FA2_ERR_ALIAS, (o, i)
        for o2 in outs:
            if o2 != o:
                assert call_bwd(fn, {o: BWD_GOOD[o2]}) == fa2.FA2_ERR_ALIAS, (o, o2)


def test_bwd_binding_checks():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fa2.backward(q, q, q, q, q, torch.zeros(1, 1, 8))


# Grouped-head backward: K/V (and dK/dV) with H_kv heads, query-head ranges
# with a partial-sum workspace
GBWD_FUNCS = ("fa2_bwd_gqa", "fa2_bwd_gqa_o32")
GBWD_NAMES = BWD_NAMES + ("part",)
GBWD_GOOD = {name: 0x10000000 + i * 64 * MiB for i, name in enumerate(GBWD_NAMES)}


def call_gbwd(fn, ptrs=None, B=1, H=8, H_kv=2, N=64, d=64, scale=0.125,
              causal=1, n_gsplits=2):
    p = dict(GBWD_GOOD)
    p.update(ptrs or {})
    return fa2.raw_call_bwd_gqa(fn, [p[n] for n in BWD_NAMES], B, H, H_kv, N, d,
                                scale, causal, n_gsplits, p["part"])


@pytest.mark.parametrize("fn", GBWD_FUNCS)
def test_bwd_gqa_validation(L, fn):
    for kw in (dict(H_kv=0), dict(H_kv=3), dict(H=2, H_kv=4), dict(n_gsplits=0),
               dict(n_gsplits=5), dict(H_kv=8, n_gsplits=2), dict(N=0)):
        assert call_gbwd(fn, **kw) == fa2.FA2_ERR_SHAPE, kw
    for name in GBWD_NAMES:
        assert call_gbwd(fn, {name: None}) == fa2.FA2_ERR_NULL, name
    # one range: no workspace needed
    assert call_gbwd(fn, {"part": None, "q": None}, n_gsplits=1) == fa2.FA2_ERR_NULL
    assert call_gbwd(fn, d=96) == fa2.FA2_ERR_HEADDIM
    assert call_gbwd(fn, scale=float("nan")) == fa2.FA2_ERR_SCALE
    for name in GBWD_NAMES:
        assert call_gbwd(fn, {name: GBWD_GOOD[name] + 4}) == fa2.FA2_ERR_ALIGN, name
    # the workspace against every other buffer; dk/dv spans are H_kv heads
    for other in BWD_NAMES:
        assert call_gbwd(fn, {"part": GBWD_GOOD[other] + 16}) == fa2.FA2_ERR_ALIAS, other
    # k is 1*2*64*64 bf16 = 16 KiB: dq right after it is fine, inside it is not
    assert call_gbwd(fn, {"dq": GBWD_GOOD["k"] + 16 * 1024 - 16}) == fa2.FA2_ERR_ALIAS
    # workspace = 2 * 2 * (1*2*64*64) fp32 = 128 KiB
    assert call_gbwd(fn, {"dv": GBWD_GOOD["part"] + 128 * 1024 - 16}) == fa2.FA2_ERR_ALIAS


def test_default_gsplits():
    # B * H_kv * key blocks = 2 * 2 * 64 = 256 units -> 4 ranges of a group of 8
    assert fa2.default_gsplits(2, 16, 2, 8192) == 4
    # never more ranges than query heads per K/V head
    assert fa2.default_gsplits(1, 4, 1, 1024) == 4
    assert fa2.default_gsplits(1, 4, 4, 1024) == 1
    # already enough workgroups
    assert fa2.default_gsplits(8, 32, 8, 16384) == 1


# Grouped-query forward: H_kv K/V heads
GQA_FUNCS = ("fa2_fwd_gqa", "fa2_fwd_gqa_o32")


def call_gqa(fn, H=4, H_kv=2, **kw):
    a = dict(GOOD)
    a.update(kw)
    return fa2.raw_call(fn, a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                        H, a["N"], a["d"], a["scale"], a["causal"], H_kv=H_kv)


@pytest.mark.parametrize("fn", GQA_FUNCS)
def test_gqa_validation(L, fn):
    for H, H_kv in ((4, 0), (4, -1), (4, 3), (2, 4), (6, 4)):
        assert call_gqa(fn, H, H_kv) == fa2.FA2_ERR_SHAPE, (H, H_kv)
    for key in ("q", "k", "v", "o"):
        assert call_gqa(fn, **{key: None}) == fa2.FA2_ERR_NULL, key
    assert call_gqa(fn, d=96) == fa2.FA2_ERR_HEADDIM
    assert call_gqa(fn, scale=float("nan")) == fa2.FA2_ERR_SCALE
    assert call_gqa(fn, v=GOOD["v"] + 8) == fa2.FA2_ERR_ALIGN
    # K and V spans are B*H_kv*N*d elements: o right after the end of k
    # (1*2*64*64 bf16 = 16 KiB) is fine only if it does not overlap
    assert call_gqa(fn, o=GOOD["k"] + 16 * 1024 - 16) == fa2.FA2_ERR_ALIAS
    assert call_gqa(fn, lse=GOOD["v"] + 4096) == fa2.FA2_ERR_ALIAS


# Split-KV forward: separate query / key lengths, key ranges + merge
SPLIT_FUNCS = ("fa2_fwd_splitkv", "fa2_fwd_splitkv_o32")
SPLIT_NAMES = ("q", "k", "v", "o", "lse", "o_part", "lse_part")
SPLIT_GOOD = {n: 0x10000000 + i * 64 * MiB for i, n in enumerate(SPLIT_NAMES)}


def call_split(fn, ptrs=None, B=1, H=4, H_kv=2, Nq=16, Nk=1000, d=128,
               scale=0.1, causal=1, n_splits=4):
    p = dict(SPLIT_GOOD)
    p.update(ptrs or {})
    return fa2.raw_call_splitkv(fn, [p[n] for n in SPLIT_NAMES], B, H, H_kv, Nq,
                                Nk, d, scale, causal, n_splits)


@pytest.mark.parametrize("fn", SPLIT_FUNCS)
def test_splitkv_validation(L, fn):
    for kw in (dict(Nq=0), dict(Nk=0), dict(H_kv=3), dict(n_splits=0),
               dict(n_splits=-2), dict(n_splits=fa2.MAX_SPLITS + 1),
               dict(B=1 << 14, H=1 << 14, Nq=1 << 10, n_splits=1000)):
        assert call_split(fn, **kw) == fa2.FA2_ERR_SHAPE, kw
    for name in ("q", "k", "v", "o", "o_part", "lse_part"):
        assert call_split(fn, {name: None}) == fa2.FA2_ERR_NULL, name
    assert call_split(fn, d=80) == fa2.FA2_ERR_HEADDIM
    assert call_split(fn, scale=float("inf")) == fa2.FA2_ERR_SCALE
    for name in SPLIT_NAMES:
        assert call_split(fn, {name: SPLIT_GOOD[name] + 4}) == fa2.FA2_ERR_ALIGN, name
    # workspaces against every input and output, and against each other
    for part in ("o_part", "lse_part"):
        for other in ("q", "k", "v", "o", "lse"):
            assert call_split(fn, {part: SPLIT_GOOD[other] + 16}) == fa2.FA2_ERR_ALIAS, (part, other)
    assert call_split(fn, {"lse_part": SPLIT_GOOD["o_part"] + 64}) == fa2.FA2_ERR_ALIAS


def call_noalloc(ptrs=None, B=1, H=4, H_kv=2, Nq=16, Nk=1000, d=128,
                 scale=0.1, causal=1, n_splits=4):
    p = dict(SPLIT_GOOD)
    p.update(ptrs or {})
    return int(fa2.lib().fa2_fwd_splitkv_noalloc(
        *[p[n] for n in SPLIT_NAMES[:5]], B, H, H_kv, Nq, Nk, d,
        ctypes.c_float(scale), causal, n_splits, None))


def test_splitkv_noalloc_validation(L):
    """The allocation-free split-KV entry point validates like
    fa2_fwd_splitkv, and a problem whose partials exceed the static
    workspace is refused with FA2_ERR_WORKSPACE on the host, before any HIP
    call."""
    for kw in (dict(Nq=0), dict(Nk=0), dict(H_kv=3), dict(n_splits=0),
               dict(n_splits=fa2.MAX_SPLITS + 1)):
        assert call_noalloc(**kw) == fa2.FA2_ERR_SHAPE, kw
    for name in ("q", "k", "v", "o"):
        assert call_noalloc({name: None}) == fa2.FA2_ERR_NULL, name
    assert call_noalloc(d=80) == fa2.FA2_ERR_HEADDIM
    assert call_noalloc(scale=float("nan")) == fa2.FA2_ERR_SCALE
    assert call_noalloc({"o": SPLIT_GOOD["o"] + 4}) == fa2.FA2_ERR_ALIGN
    assert call_noalloc({"o": SPLIT_GOOD["q"] + 16}) == fa2.FA2_ERR_ALIAS
    # n_splits * B * H * Nq * (d + 1) * 4 bytes against the 32 MiB array
    lim = fa2.NOALLOC_WORKSPACE_BYTES
    rows_ok = lim // (4 * 129 * 4)          # n_splits = 4, d = 128
    assert 4 * rows_ok * 129 * 4 <= lim < 4 * (rows_ok + 1) * 129 * 4
    big = dict(B=1, H=rows_ok + 1, H_kv=1, Nq=1, Nk=1000, n_splits=4)
    assert call_noalloc(**big) == fa2.FA2_ERR_WORKSPACE
    assert call_noalloc(B=1, H=1, H_kv=1, Nq=1 << 16, Nk=1 << 16,
                        n_splits=2) == fa2.FA2_ERR_WORKSPACE
    assert "workspace" in fa2.strerror(fa2.FA2_ERR_WORKSPACE)


def test_default_splits():
    # decode (blocks of fewer than 128 rows): about 512 workgroups, ranges of
    # at least 32 key tiles
    assert fa2.default_splits(8, 32, 1, 16384, 128) == 2
    assert fa2.default_splits(1, 1, 1, 65536, 128) == 64  # one head: 64 ranges of 16 tiles
    # grouped decode: a group's query heads share one block
    assert fa2.default_splits(8, 32, 1, 16384, 128, 8, True) == 8
    assert fa2.default_splits(1, 32, 1, 65536, 128, 8, True) == 32
    # a causal mask over several queries keeps the heads apart
    assert fa2.default_splits(8, 32, 4, 16384, 128, 8, True) == 2
    assert fa2.default_splits(8, 32, 1, 16384, 128, 4, True) == 8
    # few blocks: at least about 256 workgroups, ranges down to 16 tiles
    assert fa2.default_splits(2, 32, 16, 16384, 128, 8, False) == 16
    # short keys: never a range below the minimum length
    assert fa2.default_splits(1, 1, 1, 300, 128) == 1
    # full blocks: about 512 workgroups, ranges of at least four tiles
    assert fa2.default_splits(1, 2, 130, 4096, 128) == 16
    assert fa2.default_splits(1, 16, 512, 32768, 128) == 8
    assert fa2.default_splits(2, 32, 128, 16384, 128) == 8
    assert fa2.default_splits(1, 16, 2048, 16384, 128) == 2
    # already enough workgroups: no split
    assert fa2.default_splits(2, 16, 8192, 8192, 128) == 1
    assert fa2.default_splits(4, 32, 1024, 8192, 128, 8, True) == 1


def test_fp8_validation(L):
    Lb = fa2.lib()
    X, C, E, S = (0x10000000 + i * 64 * MiB for i in range(4))
    qz = lambda **kw: Lb.fa2_quantize_fp8(*[kw.get(n, v) for n, v in (
        ("x", X), ("codes", C), ("exps", E))], kw.get("B", 1), kw.get("H", 2),
        kw.get("N", 100), kw.get("d", 128), kw.get("R", 64), kw.get("signs", S), None)
    assert qz(x=None) == fa2.FA2_ERR_NULL and qz(exps=None) == fa2.FA2_ERR_NULL
    assert qz(R=32) == fa2.FA2_ERR_SHAPE and qz(N=0) == fa2.FA2_ERR_SHAPE
    assert qz(d=96) == fa2.FA2_ERR_HEADDIM
    assert qz(codes=C + 8) == fa2.FA2_ERR_ALIGN and qz(exps=E + 2) == fa2.FA2_ERR_ALIGN
    assert qz(codes=X + 64) == fa2.FA2_ERR_ALIAS and qz(exps=C + 64) == fa2.FA2_ERR_ALIAS
    P = [0x10000000 + i * 64 * MiB for i in range(8)]  # q8 qe k8 ke v8 ve o lse
    for fn in ("fa2_fwd_fp8", "fa2_fwd_fp8_o32"):
        f = getattr(Lb, fn)
        call = lambda ptrs, N=100, d=128, scale=0.1: f(*ptrs, 1, 2, N, d, scale, 1, 1, None)
        for i in range(7):
            bad = list(P)
            bad[i] = None
            assert call(bad) == fa2.FA2_ERR_NULL, (fn, i)
        assert call(P, d=32) == fa2.FA2_ERR_HEADDIM
        assert call(P, scale=float("nan")) == fa2.FA2_ERR_SCALE
        bad = list(P); bad[1] += 2
        assert call(bad) == fa2.FA2_ERR_ALIGN
        bad = list(P); bad[6] = P[1]          # o over q's exponents
        assert call(bad) == fa2.FA2_ERR_ALIAS
        bad = list(P); bad[6] = P[0] + 64     # o over q's codes
        assert call(bad) == fa2.FA2_ERR_ALIAS
