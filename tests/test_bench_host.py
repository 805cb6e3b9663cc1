"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the byte and
flop accounting of the workloads, and the rule that HBM traffic is reported
only from a counter summary taken on the current kernel source."""
import os

import pytest

import bench
from exact_io_aware_24_amd import inputs as wl


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_bad_step_counts_are_refused():
    assert bench.main(["--steps", "0"]) == 2
    assert bench.main(["--warmup", "-1"]) == 2


@pytest.mark.parametrize("B,H,N,d,expected", [
    # Q, K, V read and O written in bf16 plus lse in fp32, worked out by hand:
    # B=2 H=16 N=8192 d=128: 4 * 2*16*8192*128 * 2 B + 2*16*8192 * 4 B
    (2, 16, 8192, 128, 4 * 2 * 16 * 8192 * 128 * 2 + 2 * 16 * 8192 * 4),
    (4, 32, 4096, 128, 538968064),
    (8, 16, 2048, 64, 4 * 8 * 16 * 2048 * 64 * 2 + 8 * 16 * 2048 * 4),
])
def test_compulsory_bytes(B, H, N, d, expected):
    assert bench.compulsory_bytes(B, H, N, d) == expected


def test_compulsory_bytes_decode_and_shared_heads():
    # one query row against 16384 keys: K and V dominate
    got = bench.compulsory_bytes(8, 32, 16384, 128, Nq=1)
    kv = 2 * 8 * 32 * 16384 * 128 * 2
    q_o = 2 * 8 * 32 * 1 * 128 * 2
    assert got == kv + q_o + 8 * 32 * 1 * 4
    # two K/V heads shared by 16 query heads: K and V read once per K/V head
    got = bench.compulsory_bytes(2, 16, 8192, 128, H_kv=2)
    assert got == (2 * 16 * 8192 * 128 * 2 * 2 + 2 * 2 * 2 * 8192 * 128 * 2
                   + 2 * 16 * 8192 * 4)


def test_score_matrix_bytes_headline():
    # bf16 S of the headline workload: 2 * 16 * 8192^2 * 2 B = 4 GiB
    assert bench.score_matrix_bytes(2, 16, 8192) == 4 * 1024 ** 3


def test_code_only_ignores_comments_and_blank_lines():
    a = "int x = 1;  // one\n\n/* block\n comment */int y = 2;\n"
    b = "int x = 1;\nint y = 2;"
    assert bench.code_only(a) == b
    assert bench.code_only(a + "// trailing\n") == b


def test_kernel_hash_is_stable_and_distinguishes_passes():
    h1 = bench.kernel_source_hash("fwd")
    assert h1 == bench.kernel_source_hash("fwd")
    assert len(h1) == 16
    assert h1 != bench.kernel_source_hash("bwd")


def _summary(tmp_path, name, sha, fetch=100.0, write=20.0):
    p = tmp_path / ("counters_fa2_fwd_bf16_%s.md" % name)
    p.write_text("# counters\n\n- kernel_source_sha256: `%s`\n"
                 "- fetch_bytes_per_launch: %s\n- write_bytes_per_launch: %s\n"
                 % (sha, fetch, write))
    return p


def test_traffic_only_from_a_summary_of_the_current_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    cur = bench.kernel_source_hash("fwd")
    _summary(tmp_path, "now", cur)
    _summary(tmp_path, "stale", "0" * 16)
    assert bench.read_traffic("now") == 120.0
    assert bench.read_traffic("stale") is None
    assert bench.read_traffic("missing") is None


def test_committed_headline_summaries_name_their_kernel_source():
    """Every committed counter summary names the kernel source it was taken
    on, and those of the headline forward workload give fetch and write
    bytes whose sum is at least the compulsory bytes (nothing can move
    fewer) and far below the score matrix that is never written."""
    w = wl.WORKLOADS[wl.HEADLINE]
    path = os.path.join(bench.PROFILES,
                        "counters_fa2_fwd_bf16_%s.md" % wl.HEADLINE)
    text = open(path).read()
    assert "kernel_source_sha256" in text
    vals = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    total = float(vals["fetch_bytes_per_launch"]) + float(vals["write_bytes_per_launch"])
    comp = bench.compulsory_bytes(w.B, w.H, w.N, w.d)
    assert comp <= total < 0.25 * bench.score_matrix_bytes(w.B, w.H, w.N)
