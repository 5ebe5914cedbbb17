"""Sanitizer builds of the host-side code, run on the CPU.

* The fp64 oracle (oracle/gla_oracle.c) with gcc's AddressSanitizer and
  UndefinedBehaviorSanitizer, driven by tests/sanitize/oracle_main.c through
  every entry point (optional arguments present and absent, several thread
  counts, empty sequences and batches, argument errors).
* The library's host code (validation, planning, the C ABI's argument
  checks) built with the same sanitizers on the host side only
  (-Xarch_host; the device code is compiled as usual but never launched),
  driven by tests/sanitize/abi_main.cpp over every path's workspace query on
  a grid of shapes, dtypes and configs and every entry point's rejections.

Any invalid access, leak (oracle) or undefined behaviour aborts the driver
with the sanitizer's report, which the test shows.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-omit-frame-pointer",
       "-fno-sanitize-recover=all"]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, env=env, timeout=timeout)
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    r = _run(["gcc", "-std=c11", "-O1", "-g", *SAN, "-o", exe, "oracle/gla_oracle.c",
              "tests/sanitize/oracle_main.c", "-lm", "-lpthread"])
    assert r.returncode == 0, r.stderr[-4000:]
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert "clean" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="no hipcc")
def test_library_host_code_under_address_and_ub_sanitizers(tmp_path):
    host_san = [f for s in SAN for f in ("-Xarch_host", s)]
    common = ["--offload-arch=gfx950", "-std=c++17", "-g", "-I", "include",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Xarch_host", "-O1", "-Xarch_device", "-O1", *host_san]
    srcs = sorted(glob.glob(os.path.join(ROOT, "chunkwise_linear_rnn_gla_amd", "csrc", "*.hip")))
    srcs.append(os.path.join(ROOT, "tests", "sanitize", "abi_main.cpp"))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = _run([HIPCC, *common, "-c", src, "-o", obj])
        assert r.returncode == 0, f"{src}:\n{r.stderr[-4000:]}"
        return obj

    with cf.ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_san")
    r = _run([HIPCC, "--offload-arch=gfx950", *host_san, *objs, "-o", exe])
    assert r.returncode == 0, r.stderr[-4000:]
    # leaks are not checked here: the HIP runtime the library links keeps
    # allocations of its own until exit
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert "clean" in r.stdout
