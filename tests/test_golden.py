"""Values printed on the pages (fixtures under tests/golden/, each citing
its page and section)."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def _read(name):
    vals = {}
    for line in open(os.path.join(HERE, "golden", name)):
        line = line.strip()
        if line and not line.startswith("#"):
            key, val = line.split()
            vals[key] = float(val)
    return vals


def test_score_matrix_size_at_32k():
    """The bench's accounting of the score matrix that is never written
    (one head, 2-byte elements) reproduces the page's 2 GB at N = 32,000."""
    import bench
    g = _read("score_matrix_size.txt")
    got = bench.score_matrix_bytes(1, 1, int(g["seq_len"]), elem_bytes=2)
    assert abs(got - g["approx_bytes"]) <= g["rel_tol"] * g["approx_bytes"]
