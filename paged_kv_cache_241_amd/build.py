"""Build libpa.so in-tree for gfx950 (hipcc) - always recompiles.

    python -m paged_kv_cache_241_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")
ARCH = "gfx950"

# Packed-FP32 instructions are not formed (-packed-fp32-ops).  MFMA operands
# and results stay in ordinary VGPRs (no copies to and from AGPRs around the
# accumulator's VALU rescale).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-Wall", "-Wno-unused-function"]
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    """Compile the kernels and the C ABI into ``paged_kv_cache_241_amd/libpa.so``."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    jobs = [
        [hipcc, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "kernels.hip"),
         "-o", os.path.join(BUILD, "kernels.o")],
        [hipcc, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "swap.hip"),
         "-o", os.path.join(BUILD, "swap.o")],
        [hipcc, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "decode_shared.hip"),
         "-o", os.path.join(BUILD, "decode_shared.o")],
        [hipcc, *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, "pa_api.cpp"),
         "-o", os.path.join(BUILD, "pa_api.o")],
        [hipcc, *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, "block_allocator.cpp"),
         "-o", os.path.join(BUILD, "block_allocator.o")],
        [hipcc, *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, "vmm.cpp"),
         "-o", os.path.join(BUILD, "vmm.o")],
    ]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-o", tmp,
          os.path.join(BUILD, "kernels.o"), os.path.join(BUILD, "swap.o"),
          os.path.join(BUILD, "decode_shared.o"), os.path.join(BUILD, "pa_api.o"),
          os.path.join(BUILD, "block_allocator.o"), os.path.join(BUILD, "vmm.o")], verbose)
    os.replace(tmp, LIB)
    # a C caller of the ABI for the tests (plain C99 and the HIP runtime; it
    # finds libpa.so next to the package through its run path)
    c_src = os.path.join(ROOT, "tests", "c_abi_decode.c")
    cc = shutil.which("gcc") or shutil.which("cc")
    if os.path.exists(c_src) and cc:
        rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))
        _run([cc, "-std=c99", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
              "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"), c_src,
              "-o", os.path.join(ROOT, "tests", "c_abi_decode"),
              "-L", PKG, "-lpa", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
              "-Wl,-rpath,$ORIGIN/../paged_kv_cache_241_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")],
             verbose)
    # the benchmark's achievable-bandwidth probe (not part of the library)
    probe_src = os.path.join(ROOT, "bench_read_probe.hip")
    if os.path.exists(probe_src):
        _run([hipcc, "-O3", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", probe_src, "-o", os.path.join(ROOT, "bench_read_probe")], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
