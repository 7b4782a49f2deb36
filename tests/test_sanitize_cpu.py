"""Host sanitizer runs (CPU only): the oracle and the C-ABI shell built with
AddressSanitizer and UndefinedBehaviorSanitizer, each driven by a C program
under tests/sanitize/ over small inputs, degenerate cases and extreme shapes.
An out-of-bounds access, a leak (oracle), a signed overflow or a misaligned
access aborts the driver with a non-zero exit.  Only host code is
instrumented: device code is built as usual and never runs here."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "decode_kv_cache_beacon_amd", "csrc")
ROCM = "/opt/rocm"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_drive")
    _run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp",
          os.path.join(ROOT, "oracle", "beacon_oracle.c"), os.path.join(HERE, "oracle_drive.c"),
          "-lm", "-o", exe])
    r = _run([exe], env=ENV, timeout=120)
    assert "all calls clean" in r.stdout


@pytest.mark.skipif(not os.path.exists(f"{ROCM}/bin/hipcc"), reason="needs hipcc")
def test_abi_shell_under_address_and_undefined_sanitizers(tmp_path):
    """Every library source compiled with the host side instrumented (the
    sanitizer flags apply to the host pass only), linked with the driver."""
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        _run([f"{ROCM}/bin/hipcc", *flags, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    clang = f"{ROCM}/llvm/bin/clang"
    drv = str(tmp_path / "abi_drive.o")
    _run([clang, "-std=c99", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(HERE, "abi_drive.c"), "-o", drv])
    exe = str(tmp_path / "abi_drive")
    _run([clang + "++", "-fsanitize=address,undefined", *objs, drv, f"-L{ROCM}/lib",
          "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe])
    r = _run([exe], env=ENV, timeout=120)
    assert "all calls clean" in r.stdout
