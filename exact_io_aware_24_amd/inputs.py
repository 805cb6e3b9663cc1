"""Seeded synthetic attention inputs.

This module holds the workload shapes and the random-input recipe, and
nothing of the attention arithmetic: both the GPU library's tests and the
CPU oracle's tests draw their Q, K, V from here, and nothing else is shared
between the two.

The pages measure on no dataset; the workloads are synthetic by design:

* Q, K, V are drawn as ``torch.randn`` in float32 from a CPU generator
  seeded once per call (default seed 1234), in the order q, k, v (K and V
  with H_kv heads when the workload shares K/V heads between query heads);
* the outlier workload additionally picks, for Q and then for K, for every
  (batch, head) in order, ``floor(0.05 * N)`` distinct rows with
  ``torch.randperm`` from the same generator and multiplies those whole rows
  by 20 (V is left alone);
* the result is rounded to bfloat16 (round-to-nearest-even, torch's
  ``.to``) for the bf16 workloads; the tiny exactness case stays float32.

The same seed therefore gives bit-identical inputs on every machine with the
same torch version.
"""
from __future__ import annotations

import dataclasses
import math

import torch

DEFAULT_SEED = 1234


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention problem: ``[B, H, N, d]`` Q/K/V, optional causal mask."""
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    dtype: str  # "bf16" or "fp32": the type Q, K, V are stored in
    outliers: bool = False  # 5 % of Q and K rows scaled by 20
    H_kv: int = 0  # K/V heads (grouped-query attention); 0 means H
    Nq: int = 0    # query rows when they differ from the N keys; 0 means N

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        """Algorithmic FLOPs, 4*B*H*Nq*N*d, halved when causal (square)."""
        f = 4.0 * self.B * self.H * self.q_rows * self.N * self.d
        return f / 2 if self.causal else f

    @property
    def kv_heads(self) -> int:
        return self.H_kv or self.H

    @property
    def q_rows(self) -> int:
        return self.Nq or self.N

    def describe(self) -> str:
        return "B=%d,H=%d%s,%sN=%d,d=%d,%s,%s%s" % (
            self.B, self.H,
            (",H_kv=%d" % self.kv_heads) if self.kv_heads != self.H else "",
            ("Nq=%d," % self.q_rows) if self.q_rows != self.N else "",
            self.N, self.d,
            "causal" if self.causal else "non-causal", self.dtype,
            ",5%-rows-x20-outliers" if self.outliers else "")


# The five workloads.  The tiny float32 case checks exactness; the causal
# N=8192, d=128 case is the headline throughput workload.
WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32_n128_d64", 1, 1, 128, 64, False, "fp32"),
        Workload("train_b8h16_n2048_d64", 8, 16, 2048, 64, False, "bf16"),
        Workload("causal_b2h16_n8192_d128", 2, 16, 8192, 128, True, "bf16"),
        Workload("longseq_causal_b1h16_n32768_d128", 1, 16, 32768, 128, True, "bf16"),
        Workload("outlier_b4h32_n4096_d128", 4, 32, 4096, 128, False, "bf16",
                 outliers=True),
        # grouped-query attention: the headline shape with 8 query heads per
        # K/V head
        Workload("gqa_causal_b2h16kv2_n8192_d128", 2, 16, 8192, 128, True,
                 "bf16", H_kv=2),
        # decoding one token against a 16384-entry key/value cache
        Workload("decode_b8h32_nq1_nk16384_d128", 8, 32, 16384, 128, False,
                 "bf16", Nq=1),
        # the same with 4 query heads per K/V head (grouped-query decoding)
        Workload("decode_gqa_b8h32kv8_nq1_nk16384_d128", 8, 32, 16384, 128, False,
                 "bf16", H_kv=8, Nq=1),
    ]
}
HEADLINE = "causal_b2h16_n8192_d128"


def make_inputs(B: int, H: int, N: int, d: int, dtype: str = "bf16",
                seed: int = DEFAULT_SEED, outliers: bool = False, H_kv: int = 0,
                Nq: int = 0):
    """Return CPU tensors ``(q, k, v)``: q ``[B, H, Nq, d]``, k and v
    ``[B, H_kv, N, d]`` (``H_kv`` = 0 means H, ``Nq`` = 0 means N)."""
    if dtype not in ("bf16", "fp32"):
        raise ValueError("dtype must be 'bf16' or 'fp32'")
    hk = H_kv or H
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    q = torch.randn(B, H, Nq or N, d, generator=g, dtype=torch.float32)
    k = torch.randn(B, hk, N, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, hk, N, d, generator=g, dtype=torch.float32)
    if outliers:
        for t in (q, k):
            n_out = int(math.floor(0.05 * t.shape[2]))
            for b in range(B):
                for h in range(t.shape[1]):
                    rows = torch.randperm(t.shape[2], generator=g)[:n_out]
                    t[b, h, rows] *= 20.0
    if dtype == "bf16":
        q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    return q, k, v


def make_signs(d: int, seed: int = DEFAULT_SEED + 2):
    """Random +-1 signs (float32, CPU) of the FP8 path's incoherent
    processing rotation diag(signs) H / sqrt(d)."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    return (torch.randint(0, 2, (d,), generator=g) * 2 - 1).to(torch.float32)


def make_dout(B: int, H: int, N: int, d: int, seed: int = DEFAULT_SEED + 1):
    """An incoming gradient of the output for the backward pass: bf16 CPU
    tensor ``[B, H, N, d]`` of seeded standard normal values."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    return torch.randn(B, H, N, d, generator=g, dtype=torch.float32).to(torch.bfloat16)


def workload_inputs(w: Workload, seed: int = DEFAULT_SEED):
    """Inputs of a named workload (CPU tensors)."""
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, seed=seed,
                       outliers=w.outliers, H_kv=w.H_kv, Nq=w.Nq)
