"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C-ABI layer (fa2_api.cpp: argument validation, aliasing checks,
  dispatch, error codes) is built with g++ and both sanitizers against a
  host-only stand-in for the HIP runtime header and stub kernel launchers
  (tests/sanitize/), and driven through valid and invalid calls of every
  entry point: each valid call must reach exactly one launcher, each invalid
  one must return its code without launching, and the sanitizers must stay
  silent.  The bf16 forward launcher records its arguments, so the host's
  packing of grouped short query blocks (which calls run the query heads of
  a K/V head as one block, and which stay unpacked) is checked as well.
* The fp64 oracle (oracle/attn_oracle.c) is built with gcc and both
  sanitizers and every oracle pin runs against that build in a child
  process with the AddressSanitizer runtime preloaded.
No GPU code is built or run here."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def have(tool):
    return shutil.which(tool) is not None


@pytest.mark.skipif(not have("g++"), reason="g++ not available")
def test_abi_layer_under_sanitizers(tmp_path):
    exe = tmp_path / "abi_driver"
    cmd = ["g++", "-std=c++17"] + SAN + [
        "-I" + os.path.join(HERE, "sanitize"),            # host-only HIP stand-in
        "-I" + os.path.join(ROOT, "include"),
        "-I" + os.path.join(ROOT, "exact_io_aware_24_amd", "csrc"),
        os.path.join(ROOT, "exact_io_aware_24_amd", "csrc", "fa2_api.cpp"),
        os.path.join(HERE, "sanitize", "abi_driver.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    assert out.startswith("ok:"), out


@pytest.mark.skipif(not have("gcc"), reason="gcc not available")
def test_oracle_pins_under_sanitizers(tmp_path):
    import oracle
    lib = tmp_path / "liboracle_san.so"
    src = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")
    subprocess.run(["gcc", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-pthread"] + SAN + [src, "-o", str(lib), "-lm"],
                   check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    ubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True,
                           text=True, check=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("AddressSanitizer runtime not found")
    script = (
        "import sys\n"
        "sys.path[:0] = [%r, %r]\n"
        "import oracle\n"
        "from oracle_pins import ALL_PINS\n"
        "orc = oracle.OracleLib(%r)\n"
        "for pin in ALL_PINS:\n"
        "    pin(orc)\n"
        "    print('pin ok', pin.__name__, flush=True)\n"
        "print('all pins ok', len(ALL_PINS))\n" % (ROOT, HERE, str(lib)))
    preload = asan + ((":" + ubsan) if os.path.isabs(ubsan) and os.path.exists(ubsan) else "")
    env = dict(os.environ, LD_PRELOAD=preload,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True,
                       env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "all pins ok" in out, out[-4000:]
