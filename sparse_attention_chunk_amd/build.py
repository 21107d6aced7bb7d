"""Builds libfm.so (the HIP kernels and the C ABI) in-tree for gfx950.

python sparse_attention_chunk_amd/build.py [--isa DIR]

(run as a script: importing the package needs a built, current libfm.so)

--isa DIR also writes the device assembly of every source into DIR (for
register/spill inspection); the library itself is built the same way.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfm.so")
SOURCES = ["fm_api.hip", "fm_query.hip", "fm_score.hip", "fm_score_fp8.hip", "fm_select.hip", "fm_subset.hip", "fm_resident.hip", "fm_mask.hip"]
ARCH = "gfx950"

# Packed fp32 vector ops stay off for every HIP file.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # MFMA accumulators in VGPRs: the epilogue reads them every tile
                "-mllvm", "--amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfm)")


def build(isa_dir: str | None = None, verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
           "-Wno-unused-result", *DEVICE_FLAGS, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"libfm build failed:\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs)
    os.replace(tmp, LIB)
    if isa_dir:
        os.makedirs(isa_dir, exist_ok=True)
        for s in srcs:
            out = os.path.join(isa_dir, os.path.basename(s).replace(".hip", ".s"))
            subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", *DEVICE_FLAGS, "-I", INCLUDE,
                            "-I", CSRC, "--cuda-device-only", "-S", s, "-o", out], check=True,
                           capture_output=True)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--isa", default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.isa, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
