"""Ahead-of-time build of the HIP library for gfx950 (MI355X): one shared object with the C ABI
of include/dsa_indexer.h.  Run ``python -m sparse_attention_indexer_rmsnorm_amd.build``."""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdsa_indexer.so")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # no packed-fp32 instructions anywhere in the device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # MFMA results in arch VGPRs: the epilogue reads them with plain VALU ops
           "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           "-Wall", "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"),
           "-o", LIB + ".tmp"] + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (res.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
