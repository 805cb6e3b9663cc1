#!/usr/bin/env python3
"""Throughput of the exact-attention forward kernel on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one call of ``fa2_fwd`` (bf16 in, bf16 out, with lse) on the
headline workload B=2, H=16, N=8192, d=128, causal, inputs resident in HBM
(``--entry fa2_fwd_o32`` times the fp32-output sibling, ``--workload`` and
``--seq-len`` pick another shape).  ``--pass bwd`` times ``fa2_bwd`` instead
(gradients for a seeded dO, after one forward call that provides O and lse),
counted at the usual 2.5x the forward's flop: the five products S, dP, dV,
dK, dQ; with shared K/V heads it times ``fa2_bwd_gqa`` (``--gsplits`` sets
the query-head ranges per K/V head).  Workloads with fewer query rows than keys (decoding) run through
``fa2_fwd_splitkv`` with its default key-range split and are reported
against the HBM roofline (their bytes: K, V, Q read, O and lse written).
``--entry fa2_fwd_fp8`` times the FP8 attention on inputs quantised (with
the random-sign rotation of Q and K) before the timed region, against the
fp8 MFMA peak; the quantisation time of Q, K and V is reported beside it.
W untimed warm-up steps are followed by exactly K timed steps between HIP
events on the stream the kernel is launched on.  Rank 0 prints one JSON line:
TFLOP/s (4*B*H*N^2*d, halved for causal), the roofline of the kernel against
the bf16 dense MFMA peak, the HBM traffic measured by rocprofv3 counters
(when the committed counter summary matches the current kernel source), and
the fp64 CPU oracle timed on a bounded sample of the same workload.

``--per-call`` adds the median and minimum of single calls, each between its
own pair of HIP events; ``--cold-mall MiB`` writes that much scratch memory
between those calls so that the inputs are not left in the 256 MB
last-level cache.

Only one GPU is used: ``--gpus`` above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published
CSRC = os.path.join(ROOT, "exact_io_aware_24_amd", "csrc")
KERNEL_SRCS = {"fwd": ("fa2_fwd_bf16.hip", "fa2_device.h"),
               "bwd": ("fa2_bwd_bf16.hip", "fa2_device.h"),
               "fp8": ("fa2_fp8.hip", "fa2_device.h")}
PROFILES = os.path.join(ROOT, "profiles")


def score_matrix_bytes(B: int, H: int, N: int, elem_bytes: int = 2) -> float:
    """Bytes of the N x N score matrix standard attention would write per
    (batch, head), summed over B*H -- what the tiled kernel never stores."""
    return float(B) * H * N * N * elem_bytes


def compulsory_bytes(B, H, N, d, in_bytes=2, out_bytes=2, lse=True,
                     Nq=None, H_kv=None) -> float:
    """Q, K, V read once, O (and lse) written once."""
    Nq = N if Nq is None else Nq
    H_kv = H if H_kv is None else H_kv
    nq = float(B) * H * Nq * d
    nkv = float(B) * H_kv * N * d
    return (nq + 2 * nkv) * in_bytes + nq * out_bytes + (float(B) * H * Nq * 4 if lse else 0)


def code_only(text: str) -> str:
    """Source text without comments, trailing blanks and empty lines, so that
    an edit of comments alone keeps a counter summary valid."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (ln.split("//", 1)[0].rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_source_hash(which: str = "fwd") -> str:
    """Hash of the code (comments excluded) of one pass's kernel sources:
    names the kernel version that a counter summary was taken on."""
    h = hashlib.sha256()
    for name in KERNEL_SRCS[which]:
        with open(os.path.join(CSRC, name)) as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload_name: str, which: str = "fwd"):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter's reading on
    a copy of known size), or None when there is none or it was taken on a
    different kernel source."""
    kind = "fwd_fp8" if which == "fp8" else which + "_bf16"
    path = os.path.join(PROFILES, "counters_fa2_%s_%s.md" % (kind, workload_name))
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.strip()
        if line.startswith("- ") and ":" in line:
            key, val = line[2:].split(":", 1)
            vals[key.strip()] = val.strip().strip("`")
    try:
        if vals.get("kernel_source_sha256") != kernel_source_hash(which):
            return None
        fetch = float(vals["fetch_bytes_per_launch"])
        write = float(vals["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None
    return fetch + write


def rocm_version() -> str:
    """ROCm release of the installation (``/opt/rocm/.info/version``)."""
    try:
        with open("/opt/rocm/.info/version") as f:
            return f.read().strip()
    except OSError:
        return "unknown"


class ClockSampler:
    """Engine (GFX) clock of the benchmarked GPU, read through amdsmi's GPU
    metrics (``current_gfxclks``: one value per XCD, averaged) while kernels
    run: the power limit lowers the clock under load, so the achieved
    fraction of the 2.4 GHz peak mixes kernel efficiency with the clock.
    The firmware refreshes these metrics every few hundred milliseconds, so
    a timed region shorter than that may only see values from before it;
    the record says how many distinct readings it got.  Every failure
    leaves the sampler disabled (``None`` in the record); it never affects
    the timing itself."""

    def __init__(self, torch, dev):
        self.samples = []
        self._read = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            handle = handles[0] if len(handles) == 1 else None
            try:  # match the torch device by PCI address
                props = torch.cuda.get_device_properties(dev)
                want = "%04x:%02x:%02x" % (props.pci_domain_id, props.pci_bus_id,
                                           props.pci_device_id)
                for h in handles:
                    if amdsmi.amdsmi_get_gpu_device_bdf(h).lower().startswith(want):
                        handle = h
            except Exception:
                pass
            if handle is None:
                return

            def read():
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                vals = [x for x in m.get("current_gfxclks", [])
                        if isinstance(x, (int, float))]
                if not vals and isinstance(m.get("current_gfxclk"), (int, float)):
                    vals = [m["current_gfxclk"]]
                return sum(vals) / len(vals) if vals else None

            read()
            self._read = read
        except Exception:
            self._read = None

    def poll_until(self, event, period_s=0.005):
        """Sample until ``event`` has completed (the kernels drained)."""
        out = []
        while not event.query():
            if self._read is not None:
                try:
                    v = self._read()
                    if v is not None:
                        out.append(float(v))
                except Exception:
                    self._read = None
            time.sleep(period_s)
        return out

    @staticmethod
    def summary(samples):
        if not samples:
            return None
        s = sorted(samples)
        return {"mean_mhz": round(sum(s) / len(s), 1), "min_mhz": round(s[0], 1),
                "max_mhz": round(s[-1], 1), "samples": len(s),
                "distinct": len(set(s)),
                "source": "amdsmi gpu metrics, current_gfxclks (mean over XCDs)"}


def cpu_baseline_bwd(w, q, k, v, do, budget_s: float):
    """Time the fp64 gradient oracle (as it stands) on whole heads of the
    workload, as many as fit the budget after timing the first one."""
    import oracle
    BH = w.B * w.H
    G = w.H // w.kv_heads  # query heads per K/V head
    qf, gf = (t.reshape(BH, w.N, w.d) for t in (q, do))
    kf, vf = (t.reshape(BH // G, w.N, w.d) for t in (k, v))
    n_heads, dt, threads = 0, 0.0, 0
    t0 = time.perf_counter()
    while n_heads < BH and (n_heads == 0 or dt * (n_heads + 1) / n_heads <= budget_s):
        h = n_heads
        _, _, _, _, threads = oracle.attention_bwd(qf[h], kf[h // G], vf[h // G],
                                                   gf[h], w.scale, w.causal)
        n_heads += 1
        dt = time.perf_counter() - t0
    flops = 2.5 * w.flops / BH * n_heads
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": "%d of %d heads (all %d rows each) of %s, backward; fp64 C "
                  "oracle, %.1f s wall, %.3g flop counted like the GPU metric"
                  % (n_heads, BH, w.N, w.describe(), dt, flops),
    }


def cpu_baseline(w, q, k, v, budget_s: float):
    """Time the fp64 oracle (as it stands) on a bounded sample of the
    workload: whole heads, all their rows, as many heads as fit the budget
    after a one-head calibration on a row subset."""
    import numpy as np
    import torch
    import oracle
    BH = w.B * w.H
    if w.kv_heads != w.H:  # grouped K/V heads: the oracle's definition
        k = torch.from_numpy(oracle.expand_kv_heads(k, w.H))
        v = torch.from_numpy(oracle.expand_kv_heads(v, w.H))
    nq = w.q_rows
    qf = q.reshape(BH, nq, w.d)
    kf, vf = (t.reshape(BH, w.N, w.d) for t in (k, v))
    off = w.N - nq  # causal: query i at key position i + off

    def head_flops(rows):
        keys = np.clip(rows + off + 1, 0, w.N) if w.causal else np.full(rows.shape, w.N)
        return float(np.sum(4.0 * w.d * keys))

    # calibration: every 16th row of head 0
    rows = np.arange(0, nq, 16, dtype=np.int64)
    t0 = time.perf_counter()
    _, _, threads = oracle.attention_rows(qf[0, rows], rows + off, kf[0], vf[0],
                                          w.scale, w.causal)
    rate = head_flops(rows) / max(time.perf_counter() - t0, 1e-9)
    all_rows = np.arange(nq, dtype=np.int64)
    per_head = head_flops(all_rows)
    n_heads = int(max(1, min(BH, round(budget_s * rate / per_head))))
    t0 = time.perf_counter()
    for h in range(n_heads):
        _, _, threads = oracle.attention_offset(qf[h:h + 1], kf[h:h + 1], vf[h:h + 1],
                                                w.scale, w.causal)
    dt = time.perf_counter() - t0
    flops = per_head * n_heads
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": "%d of %d heads (all %d query rows each) of %s; fp64 C oracle, "
                  "%.1f s wall, %.3g flop counted like the GPU metric"
                  % (n_heads, BH, nq, w.describe(), dt, flops),
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps; the engine clock needs ~0.5 s of load to settle")
    ap.add_argument("--workload", default=None,
                    help="workload name (default: the headline workload)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle time for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", default="fwd", choices=("fwd", "bwd"),
                    help="forward (fa2_fwd) or backward (fa2_bwd) pass")
    ap.add_argument("--entry", default=None,
                    choices=("fa2_fwd", "fa2_fwd_o32", "fa2_fwd_fp8", "fa2_bwd",
                             "fa2_bwd_o32"),
                    help="entry point to time (o32: fp32 outputs)")
    ap.add_argument("--seq-len", type=int, default=0,
                    help="override the workload's sequence length")
    ap.add_argument("--splits", type=int, default=0,
                    help="key ranges for fa2_fwd_splitkv workloads (0: the default)")
    ap.add_argument("--gsplits", type=int, default=0,
                    help="query-head ranges per shared K/V head for the grouped "
                         "backward (0: the default)")
    ap.add_argument("--per-call", action="store_true",
                    help="also time single calls (median, min)")
    ap.add_argument("--cold-mall", type=int, default=0, metavar="MIB",
                    help="with --per-call: write this many MiB between calls")
    ap.add_argument("--clock-window", type=float, default=2.5, metavar="S",
                    help="seconds of untimed load after the timed steps during which "
                         "the engine clock is sampled (0: none)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter "
                         "calibration runs)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print("bench.py measures one GPU only (the library has no multi-GPU "
              "path); got --gpus %d" % args.gpus, file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch
    import exact_io_aware_24_amd as fa2
    from exact_io_aware_24_amd import inputs as wl

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    name = args.workload or wl.HEADLINE
    w = wl.WORKLOADS[name]
    if w.dtype != "bf16":
        print("the benchmark times the bf16 path", file=sys.stderr)
        return 2
    if args.seq_len:
        if args.seq_len < 1:
            print("--seq-len must be >= 1", file=sys.stderr)
            return 2
        w = dataclasses.replace(w, N=args.seq_len)
    entry = args.entry or ("fa2_fwd" if args.which == "fwd" else "fa2_bwd")
    if not entry.startswith("fa2_" + args.which):
        print("--entry %s does not belong to --pass %s" % (entry, args.which),
              file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    decode = w.q_rows != w.N
    if entry == "fa2_fwd_fp8" and (decode or w.kv_heads != w.H):
        print("fa2_fwd_fp8 takes equal query and key lengths and one K/V head per "
              "query head", file=sys.stderr)
        return 2
    if decode and (args.which == "bwd" or entry != "fa2_fwd" or args.seq_len):
        print("workloads with fewer queries than keys time fa2_fwd_splitkv only",
              file=sys.stderr)
        return 2
    q, k, v = wl.make_inputs(w.B, w.H, w.N, w.d, w.dtype, outliers=w.outliers,
                             H_kv=w.H_kv, Nq=w.Nq)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    out_dtype = torch.float32 if entry.endswith("_o32") else torch.bfloat16
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
    n_splits = None
    n_gsplits = None
    fp8 = entry == "fa2_fwd_fp8"
    quant_ms = None
    if fp8:
        flops = w.flops
        signs = wl.make_signs(w.d).to(dev)
        o = torch.empty(qd.shape, dtype=torch.bfloat16, device=dev)

        def quantize():
            return (fa2.quantize_fp8(qd, 128, signs), fa2.quantize_fp8(kd, 64, signs),
                    fa2.quantize_fp8(vd, 64, None))
        (q8, qe), (k8, ke), (v8, ve) = quantize()
        for _ in range(20):
            quantize()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(50):
            quantize()
        e1.record()
        torch.cuda.synchronize()
        quant_ms = e0.elapsed_time(e1) / 50

        def step():
            fa2.forward_fp8(q8, qe, k8, ke, v8, ve, causal=w.causal, scale=w.scale,
                            rotated=True, out=o, lse=lse)
    elif decode:
        flops = w.flops
        entry = "fa2_fwd_splitkv"
        n_splits = args.splits or fa2.default_splits(w.B, w.H, w.q_rows, w.N, w.d,
                                                     w.kv_heads, w.causal)
        o = torch.empty(qd.shape, dtype=out_dtype, device=dev)
        o_part = torch.empty((n_splits,) + tuple(qd.shape), dtype=torch.float32, device=dev)
        lse_part = torch.empty((n_splits,) + tuple(qd.shape[:3]), dtype=torch.float32,
                               device=dev)

        def step():
            fa2.forward_splitkv(qd, kd, vd, causal=w.causal, scale=w.scale,
                                n_splits=n_splits, out=o, lse=lse, o_part=o_part,
                                lse_part=lse_part)
    elif args.which == "fwd":
        flops = w.flops
        o = torch.empty(qd.shape, dtype=out_dtype, device=dev)

        def step():
            fa2.forward(qd, kd, vd, causal=w.causal, scale=w.scale,
                        out_dtype=out_dtype, out=o, lse=lse)
    else:
        flops = 2.5 * w.flops
        do = wl.make_dout(w.B, w.H, w.N, w.d)
        dod = do.to(dev)
        o, _ = fa2.forward(qd, kd, vd, causal=w.causal, scale=w.scale, lse=lse)
        grads = [torch.empty(t.shape, dtype=out_dtype, device=dev) for t in (qd, kd, vd)]
        delta = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
        dkv_part = None
        if w.kv_heads != w.H:  # shared K/V heads: the grouped entry point
            entry = entry.replace("fa2_bwd", "fa2_bwd_gqa")
            n_gsplits = args.gsplits or fa2.default_gsplits(w.B, w.H, w.kv_heads, w.N)
            if n_gsplits > 1:
                dkv_part = torch.empty((2, n_gsplits) + tuple(kd.shape),
                                       dtype=torch.float32, device=dev)

        def step():
            fa2.backward(qd, kd, vd, o, dod, lse, causal=w.causal, scale=w.scale,
                         out_dtype=out_dtype, dq=grads[0], dk=grads[1],
                         dv=grads[2], delta=delta, n_gsplits=n_gsplits,
                         dkv_part=dkv_part)

    for _ in range(args.warmup):
        step()
    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
    clock = ClockSampler(torch, dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    clock_timed = clock.poll_until(end)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    tflops = flops / (ms * 1e-3) / 1e12

    per_call = None
    if args.per_call:
        scratch = (torch.empty(args.cold_mall * (1 << 20) // 4, dtype=torch.float32,
                               device=dev) if args.cold_mall else None)
        pairs = []
        for i in range(args.steps):
            if scratch is not None:
                scratch.fill_(float(i))
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        per = sorted(a.elapsed_time(b) for a, b in pairs)
        per_call = {"median_ms": round(per[len(per) // 2], 5),
                    "min_ms": round(per[0], 5),
                    "median_tflops": round(flops / (per[len(per) // 2] * 1e-3) / 1e12, 3),
                    "cold_mall_mib": args.cold_mall}

    # the clock this kernel sustains: the same step for --clock-window seconds
    # after the timed region (not timed), sampled the same way; the firmware
    # refreshes the reading about once a second, so only the samples of the
    # last 60 % of the window are kept
    clock_load = []
    if clock._read is not None and args.clock_window > 0:
        n_load = max(1, int(math.ceil(args.clock_window / max(ms * 1e-3, 1e-6))))
        n_load = min(n_load, 100000)
        done = torch.cuda.Event()
        for _ in range(n_load):
            step()
        done.record(stream)
        clock_load = clock.poll_until(done)
        torch.cuda.synchronize()
        clock_load = clock_load[int(0.4 * len(clock_load)):]

    default_entry = "fa2_fwd_splitkv" if decode else "fa2_" + args.which
    same_shape = not args.seq_len and not args.splits and not args.gsplits and \
        entry in (default_entry, "fa2_fwd_fp8", "fa2_bwd_gqa")
    traffic = read_traffic(name, "fp8" if fp8 else args.which) if same_shape else None
    comp = compulsory_bytes(w.B, w.H, w.N, w.d, Nq=w.q_rows, H_kv=w.kv_heads)
    if decode:  # bandwidth-bound: K and V are read once, little arithmetic
        gbs = comp / (ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                    "traffic": traffic}
    else:
        peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS
        roofline = {"bound": "mfma", "achieved": round(tflops, 3),
                    "peak": peak, "unit": "TFLOP/s",
                    "frac": round(tflops / peak, 4), "traffic": traffic}
    # what one timed call launches, i.e. what the HIP-event duration behind
    # roofline.achieved covers
    if decode:
        roofline_scope = ("the call launches the key-range kernel and, with n_splits > 1, "
                          "the merge kernel; achieved = compulsory bytes per call / the "
                          "call's mean duration, both kernels included (the range kernel "
                          "alone is in the rocprofv3 trace summary)")
    elif args.which == "bwd":
        roofline_scope = ("the call launches the delta, dK/dV and dQ kernels (and, for "
                          "grouped K/V heads with several ranges, the partial-sum "
                          "reductions); achieved = the five products' flop per call / the "
                          "call's mean duration (per-kernel figures are in the rocprofv3 "
                          "trace summary)")
    else:
        roofline_scope = ("the call is one kernel launch; achieved = its flop per launch / "
                          "its mean duration")
    rec = {
        "metric": "attention %s TFLOP/s (1 MI355X) and %% of bf16 MFMA peak" % args.which,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3" if fp8 else "bf16",
        "data": "synthetic (seeded randn, bf16)",
        "config": {"workload": name, "B": w.B, "H": w.H, "H_kv": w.kv_heads,
                   "Nq": w.q_rows, "N": w.N, "d": w.d, "causal": w.causal,
                   "scale": w.scale, "flops_per_step": flops, "entry_point": entry,
                   "n_splits": n_splits, "n_gsplits": n_gsplits},
        "roofline": roofline,
        "roofline_scope": roofline_scope,
        "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "score_matrix_bytes_not_written": score_matrix_bytes(w.B, w.H, w.N),
        "compulsory_hbm_bytes": comp,
        "kernel_source_sha256": kernel_source_hash("fp8" if fp8 else args.which),
        "gpu": torch.cuda.get_device_name(dev),
        "gfx_clock_during_timed_steps": clock.summary(clock_timed),
        "gfx_clock_sustained_after_timing": clock.summary(clock_load),
        "gfx_clock_note": ("amdsmi refreshes the engine clock reading about once a "
                           "second: readings during a shorter timed region may "
                           "predate it; the sustained figure is taken over the last "
                           "60 % of --clock-window seconds of the same step, untimed"),
        "rocm": rocm_version(),
        "torch": torch.__version__,
        "seed": wl.DEFAULT_SEED,
    }
    if per_call is not None:
        rec["per_call"] = per_call
    if quant_ms is not None:
        rec["fp8_quantize_ms"] = round(quant_ms, 5)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = (cpu_baseline(w, q, k, v, args.cpu_budget)
                               if args.which == "fwd" else
                               cpu_baseline_bwd(w, q, k, v, do, args.cpu_budget))
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
