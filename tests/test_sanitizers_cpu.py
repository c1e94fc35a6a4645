"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers under tests/sanitize/ are built with the sanitizers and run:

* oracle_host.c with oracle/rbq_oracle.c (gcc): every oracle entry point on
  ragged, grouped and degenerate shapes, every fp16 bit pattern;
* abi_host.c with every library source (hipcc; the sanitizers on the host
  half only, the device code is built as usual): size and shape arithmetic
  over extreme shapes, kernel-family choice, argument checks, and the program
  builder on long op lists.  No call reaches a device.

Any sanitizer report aborts the driver (-fno-sanitize-recover=all), so a
non-zero exit fails the test.
"""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

from gemm_rbq_encode_amd import build as libbuild

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN_C = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
# host-only sanitizers for hipcc: each flag applies to the host compilation
SAN_HIP = []
for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"):
    SAN_HIP += ["-Xarch_host", f]
SAN_HIP += ["-g"]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_host")
    _run(["gcc", "-O1", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", *SAN_C,
          os.path.join(ROOT, "oracle", "rbq_oracle.c"), os.path.join(HERE, "sanitize", "oracle_host.c"),
          "-lm", "-o", exe])
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=1")
    r = _run([exe], env=env)
    assert "oracle host checks passed" in r.stdout


@pytest.mark.skipif(not os.path.exists(libbuild.HIPCC), reason="hipcc not found")
def test_library_host_code_under_sanitizers(tmp_path):
    flags = [f for f in libbuild.FLAGS if f != "-O3"] + ["-O1"]

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        _run([libbuild.HIPCC, *flags, *SAN_HIP, "-c", os.path.join(libbuild.CSRC, src), "-o", obj])
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, libbuild.SOURCES))
    exe = str(tmp_path / "abi_host")
    _run([libbuild.HIPCC, "--offload-arch=gfx950", *SAN_HIP, "-I", os.path.join(ROOT, "include"),
          "-x", "c", os.path.join(HERE, "sanitize", "abi_host.c"), "-x", "none", *objs, "-o", exe])
    # leaks are not checked here: the HIP runtime keeps allocations for the
    # life of the process
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = _run([exe], env=env)
    assert "library host checks passed" in r.stdout
