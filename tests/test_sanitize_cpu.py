"""The C-ABI host code (argument validation, error reporting, model clean-up
on failure) built with AddressSanitizer and UndefinedBehaviorSanitizer on the
host side, and driven through every entry point's validation and error paths
by tests/abi_validation_driver.c (CPU only: nothing reaches the device).  The
kernels are linked from the regular build, uninstrumented; the sanitizers
apply to the host code only."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from sparse_kv_cache_value_amd import build as libbuild

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
OUT = os.path.join(libbuild.BUILD, "sanitize")


def _have_gpu() -> bool:
    import torch
    return torch.cuda.device_count() > 0


@pytest.fixture(scope="module")
def driver():
    if shutil.which(libbuild.hipcc()) is None and not os.path.exists(libbuild.hipcc()):
        pytest.skip("hipcc not found")
    if not all(os.path.exists(os.path.join(libbuild.BUILD, os.path.basename(s) + ".o"))
               for s in libbuild.sources() if s.endswith(".hip")):
        libbuild.build()
    os.makedirs(OUT, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = os.path.join(OUT, "api.cpp.o")
    drv_o = os.path.join(OUT, "driver.o")
    exe = os.path.join(OUT, "abi_validation_driver")
    cc = libbuild.hipcc()
    flags = [f"--offload-arch={libbuild.ARCH}", "-O1", "-g", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    subprocess.run([cc, *flags, *san, "-I", libbuild.CSRC, "-c", os.path.join(libbuild.CSRC, "api.cpp"), "-o", api_o],
                   check=True, capture_output=True)
    subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-I", os.path.join(ROOT, "include"), "-c", os.path.join(HERE, "abi_validation_driver.c"),
                    "-o", drv_o], check=True, capture_output=True)
    kobjs = [os.path.join(libbuild.BUILD, os.path.basename(s) + ".o") for s in libbuild.sources()
             if s.endswith(".hip")]
    subprocess.run([cc, f"--offload-arch={libbuild.ARCH}", *san, "-o", exe, drv_o, api_o, *kobjs, "-lm"],
                   check=True, capture_output=True)
    return exe


def test_validation_paths_under_sanitizers(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    arg = ["gpu"] if _have_gpu() else []
    r = subprocess.run([driver, *arg], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all validation paths as documented" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
