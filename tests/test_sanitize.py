"""The oracle and the C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on
the CPU.

- The oracle's C, built by gcc with ASan and UBSan, runs every pin.
- The HIP library, built with the same sanitizers on its host code only (the device code is
  neither instrumented nor run), runs the ABI tests: symbol exports, workspace sizes, the chunk
  planner and every host-side argument check.

Each runs in a child process with the sanitizer runtime preloaded, put in front of anything
already preloaded; any report ends the child with an error.  Planted-mistake builds of the
oracle are not run here: some of them read out of range on purpose.
"""
import glob
import os
import shlex
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}
# host-side sanitizer flags for the HIP build: each one applies to the host pass only
HOST_SAN = shlex.split("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                       "-Xarch_host -fno-sanitize-recover=undefined "
                       "-Xarch_host -fno-omit-frame-pointer")


def _child(preload: str, setup: str, args: list) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env.update(SAN_ENV)
    prior = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = preload + (":" + prior if prior else "")
    code = "\n".join([
        "import sys",
        setup,
        "import pytest",
        f"rc = pytest.main({args!r} + ['-q', '-x', '-m', 'not gpu', '-p', 'no:cacheprovider'])",
        "print('LOADED', LOADED())",
        "sys.exit(rc)",
    ])
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=900)


def _check(res: subprocess.CompletedProcess, lib: str) -> None:
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert f"LOADED {lib}" in out, out[-2000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-fopenmp",
                    "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11",
                    "-o", lib, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    setup = ("import oracle\n"
             f"oracle._LIB_PATH = {lib!r}\n"
             "LOADED = lambda: oracle.lib()._name")
    _check(_child(asan, setup, ["tests/test_oracle_pins.py"]), lib)


def test_abi_host_code_under_sanitizers(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not os.path.exists(hipcc) or not rts:
        pytest.skip("hipcc or clang's ASan runtime is not installed")
    lib = str(tmp_path / "libdsa_san.so")
    srcs = sorted(glob.glob(os.path.join(ROOT, "sparse_attention_indexer_rmsnorm_amd", "csrc",
                                         "*.hip")))
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + HOST_SAN + [
           "-I", os.path.join(ROOT, "include"), "-o", lib] + srcs
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    setup = ("import sparse_attention_indexer_rmsnorm_amd as ix\n"
             f"ix.LIB_PATH = {lib!r}\n"
             "LOADED = lambda: ix.lib()._name")
    _check(_child(rts[-1], setup, ["tests/test_abi.py"]), lib)
