"""CPU-side code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

* The oracle (`oracle/csa2_oracle.c`) is built with gcc and both sanitizers together with
  `tests/sanitize/oracle_driver.c`, which calls every oracle entry point on small seeded
  inputs (ragged batch, both key layouts, a prefill chunk, quantiser edge values).
* The library's host code (argument checks, layouts, workspace and split sizes of every
  `csrc/*.hip` file) is built with hipcc, the sanitizers on the host side only, and linked
  with `tests/sanitize/host_driver.cpp`, whose calls the library must all reject or size
  on the host; no GPU is made visible to it, so no kernel can run.

Any sanitizer report aborts the driver with a non-zero status."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = dict(ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-g", "-O1", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          os.path.join(ROOT, "oracle", "csa2_oracle.c"), os.path.join(HERE, "oracle_driver.c"),
          "-lm", "-o", exe])
    out = _run([exe], env={**os.environ, **SAN_ENV}, timeout=600)
    assert "oracle driver: ok" in out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "kv_cache_decode_csa2_amd", "csrc")
    srcs = sorted(f for f in os.listdir(csrc) if f.endswith(".hip"))
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    common = ["-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", *san,
              "-I", os.path.join(ROOT, "include"), "-I", csrc]

    def compile_one(f):
        obj = str(tmp_path / (f + ".o"))
        _run([HIPCC, "--offload-arch=gfx950", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", *common, "-c", os.path.join(csrc, f), "-o", obj])
        return obj

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "host_driver.o")
    _run([HIPCC, *common, "-c", os.path.join(HERE, "host_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "host_driver")
    _run([HIPCC, "--offload-arch=gfx950", *san, *objs, drv, "-o", exe])
    env = {**os.environ, **SAN_ENV, "HIP_VISIBLE_DEVICES": "", "ROCR_VISIBLE_DEVICES": "",
           # the HIP runtime's own allocations outlive main(); the library allocates nothing
           "ASAN_OPTIONS": "detect_leaks=0"}
    out = _run([exe], env=env, timeout=600)
    assert "host driver: ok" in out
