"""Build libpkv.so in-tree: HIP kernels for gfx950 with hipcc, host code with g++.

    python -m paged_kv_cache_prefill_amd.build

Every call compiles from scratch (the output is replaced atomically).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpkv.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs (the short-query tiles are LDS-limited to
    # one work group per CU, where the compiler would otherwise shuttle
    # accumulators between AGPRs and VGPRs inside the key loop)
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
]
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
              "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include"]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in proc.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if proc.returncode != 0:
        raise RuntimeError(f"build step failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False):
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    gxx = shutil.which("g++") or "g++"
    tmp = tempfile.mkdtemp(prefix="pkv_build_")
    try:
        hip_srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
        objs = [os.path.join(tmp, f[:-4] + ".o") for f in hip_srcs]
        hobj = os.path.join(tmp, "pkv_host.o")
        steps = [[hipcc, *HIP_FLAGS, "-c", os.path.join(CSRC, f), "-o", o]
                 for f, o in zip(hip_srcs, objs)]
        steps.append([gxx, *HOST_FLAGS, "-c", os.path.join(CSRC, "pkv_host.cpp"), "-o", hobj])
        with ThreadPoolExecutor(max_workers=min(8, len(steps))) as ex:
            outs = list(ex.map(_run, steps))
        out_tmp = os.path.join(tmp, "libpkv.so")
        outs.append(_run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, hobj,
                          "-o", out_tmp, f"-L{ROCM}/lib", "-lamdhip64"]))
        staged = LIB + ".tmp"
        shutil.copyfile(out_tmp, staged)
        os.chmod(staged, 0o755)
        os.replace(staged, LIB)
        if verbose:
            for o in outs:
                if o.strip():
                    print(o)
        return LIB
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
