"""The C-ABI shim under AddressSanitizer (CPU, no GPU needed): every libmsa
source is compiled with ASan on its host code only (-Xarch_host before each
sanitizer flag; the device code is unchanged), linked with
tests/asan/abi_host_checks.c, and run.  The driver exercises the host side
of every entry point: argument and problem checks (null, misaligned,
inconsistent, unsupported), layout and scratch queries, the grid bound, the
allocation-free backward's size limit.  Any out-of-bounds or leaked host
memory aborts the run with a sanitizer report."""
import concurrent.futures
import glob
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
COMMON = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-munsafe-fp-atomics",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    assert r.returncode == 0, "\n".join(l for l in r.stderr.splitlines() if "packed-fp32" not in l)[-3000:]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_host_paths_under_address_sanitizer():
    tmp = tempfile.mkdtemp(prefix="msa_asan_")
    try:
        srcs = sorted(glob.glob(os.path.join(ROOT, "block_sparse_attention_k2q_amd", "csrc", "*.hip")))
        jobs = [[HIPCC, *COMMON, "-std=c++17", *HOST_ASAN, "-c", s, "-o", os.path.basename(s) + ".o"]
                for s in srcs]
        jobs.append([HIPCC, "-x", "c", "-O1", "-g", *HOST_ASAN, "-I", os.path.join(ROOT, "include"), "-c",
                     os.path.join(ROOT, "tests", "asan", "abi_host_checks.c"), "-o", "driver.o"])
        with concurrent.futures.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as pool:
            for f in [pool.submit(_run, cmd, tmp) for cmd in jobs]:
                f.result()
        objs = ["driver.o"] + [os.path.basename(s) + ".o" for s in srcs]
        _run([HIPCC, "--offload-arch=gfx950", *HOST_ASAN, "-o", "abi_checks", *objs], tmp)
        env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:detect_leaks=1")
        r = subprocess.run([os.path.join(tmp, "abi_checks")], cwd=tmp, capture_output=True, text=True,
                           env=env, timeout=120)
        assert "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
        assert r.returncode == 0, r.stdout + r.stderr[-3000:]
        assert "0 failure(s)" in r.stdout
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
