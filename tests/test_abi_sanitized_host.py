"""The ABI's host code (abi.cpp: validation, split plans, workspace formulas)
built with AddressSanitizer and UndefinedBehaviorSanitizer, driven by
tests/abi_fuzz_driver.c over fixed and random arguments.

The host part is compiled with g++ on its own (no device code in it) and
linked against the built libgha.so for the launch functions, which are never
reached: the driver runs only where no HIP device is visible, so every call
stops at an argument check or at the device check after them."""
import os
import shutil
import subprocess

import pytest

import grouped_head_latent_amd as gha

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "grouped_head_latent_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None or shutil.which("gcc") is None:
        pytest.skip("g++/gcc not available")
    if not os.path.exists(gha.library_path()):
        from grouped_head_latent_amd import build
        build.build()
    out = tmp_path_factory.mktemp("sanitized")
    abi_o, drv_o, exe = str(out / "abi.o"), str(out / "driver.o"), str(out / "abi_fuzz")
    steps = [
        ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", f"{ROCM}/include", "-I", f"{ROOT}/include",
         "-c", f"{PKG}/csrc/abi.cpp", "-o", abi_o],
        ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", *SAN, "-I", f"{ROOT}/include",
         "-c", f"{ROOT}/tests/abi_fuzz_driver.c", "-o", drv_o],
        ["g++", *SAN, drv_o, abi_o, f"-L{PKG}", "-lgha", f"-Wl,-rpath,{PKG}", f"-L{ROCM}/lib", "-lamdhip64",
         f"-Wl,-rpath,{ROCM}/lib", "-o", exe],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr}"
    return exe


def run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("GHA_DEBUG_CHECKS", None)
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=300, env=env)
    if r.returncode == 77:
        pytest.skip("a HIP device is visible: the driver only runs where every call stops before a launch")
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_validation_is_clean_under_asan_and_ubsan(driver, seed):
    out = run(driver, 100000, seed)
    assert out.strip().splitlines()[-1].startswith("ok ")
    counts = dict(kv.split("=") for kv in out.split("statuses:")[1].splitlines()[0].split())
    # the random calls reach every kind of refusal, and many pass every
    # argument check and stop only at the device check
    for name in ("GHA_ERR_NULL", "GHA_ERR_SHAPE", "GHA_ERR_GROUPING", "GHA_ERR_STRIDE", "GHA_ERR_ALIGN",
                 "GHA_ERR_DTYPE", "GHA_ERR_HEAD_DIM", "GHA_ERR_WORKSPACE"):
        assert int(counts[name]) > 0, name
    assert int(counts["GHA_ERR_HIP"]) > 1000
