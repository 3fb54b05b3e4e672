"""Build ``libsmla.so`` (the GPU library) in-tree with hipcc for gfx950.

    python -m sparse_mla_decode_smla_amd.build

The library is written next to this file; the binding loads it from there.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libsmla.so")
SOURCES = [os.path.join(HERE, "csrc", f)
           for f in ("smla_plan.cpp", "smla_decode.hip", "smla_combine.hip", "smla_indexer.hip")]
INCLUDE = [os.path.join(ROOT, "include"), os.path.join(HERE, "csrc")]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return path


PROBE_PATH = os.path.join(HERE, "libsmla_probe.so")
PROBE_SOURCES = [os.path.join(HERE, "csrc", "probe_stream.hip")]


def build(verbose: bool = False) -> str:
    """Build libsmla.so (the decode library) and libsmla_probe.so (the benchmark's stream-read probe)."""
    _build_one(PROBE_SOURCES, PROBE_PATH, verbose)
    return _build_one(SOURCES, LIB_PATH, verbose)


# AddressSanitizer and UndefinedBehaviorSanitizer for the host pass only (each flag behind -Xarch_host);
# the GPU code is built as usual.  The runtime must be preloaded into the process that loads the library.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_sanitized(out_path: str, verbose: bool = False) -> str:
    """libsmla.so with its host code (plan, argument checks, launch set-up) sanitized, at out_path."""
    return _build_one(SOURCES, out_path, verbose, extra=HOST_SANITIZE)


def _build_one(sources, lib_path: str, verbose: bool, extra=()) -> str:
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", *extra,
           # packed fp32 VALU forms stay disabled in the GPU code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # MFMA results in VGPRs: the partial kernel keeps Q in AGPRs and its
           # output accumulators in VGPRs, which fits two waves per SIMD unspilled
           "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           "-Wall", "-Wno-unused-command-line-argument"]
    for inc in INCLUDE:
        cmd += ["-I", inc]
    cmd += ["-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the GPU-only feature flag; drop that notice.
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
