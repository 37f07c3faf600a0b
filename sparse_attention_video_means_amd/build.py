"""Build libsvgear.so (HIP, gfx950) in-tree.

Every ``csrc/*.hip`` file is compiled to an object with hipcc for gfx950 and
the objects are linked into ``libsvgear.so`` next to this file. Packed fp32
instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsvgear.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs: the kernels fit in 256 VGPRs and the
    # AGPR form makes the register allocator copy accumulators every tile
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]

# Extra flags per source file. The attention and probe kernels take running
# maxima of matrix-core results; with NaN inputs excluded the compiler drops
# the quieting instructions IEEE mode would otherwise put before every v_max.
# The assignment and probe kernels run vector arithmetic on every result the
# matrix cores produce; with the MFMA results in ordinary registers no
# accumulator-register read precedes it.
FILE_FLAGS = {
    "svgear_attend.hip": ["-fno-honor-nans"],
    "svgear_kmeans.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "svgear_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature flag: harmless noise
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l
                    and "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every HIP source and link libsvgear.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(BUILD, f[:-4] + ".o") for f in srcs]

    def one(i):
        cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(srcs[i], []), "-c", os.path.join(CSRC, srcs[i]),
               "-o", objs[i]]
        out = _run(cmd)
        if verbose and out.strip():
            print(out)

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(one, range(len(srcs))))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


SAN_LIB = os.path.join(BUILD, "libsvgear_san.so")
# host-only sanitizers: each -fsanitize= applies to the host pass alone, device
# code is built exactly as in the product library
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_sanitized() -> str:
    """A build of the library whose ABI layer (argument validation, workspace
    carving; csrc/svgear_api.hip) has its host code instrumented with
    AddressSanitizer and UndefinedBehaviorSanitizer. The kernels and their
    launchers are the product build's objects. Load it with the sanitizer
    runtime preloaded (asan_runtime()) and SVGEAR_LIB pointing at it."""
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(BUILD, f[:-4] + ".o") for f in srcs if f != "svgear_api.hip"]
    if not all(os.path.exists(o) for o in objs):
        build()
    api = os.path.join(BUILD, "svgear_api_san.o")
    _run([HIPCC, *[f for f in CFLAGS if f != "-O3"], "-O1", "-g", *SAN_FLAGS, "-c",
          os.path.join(CSRC, "svgear_api.hip"), "-o", api])
    tmp = SAN_LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host",
          "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o",
          tmp, api, *objs])
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def asan_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of the HIP toolchain."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm")
    return hits[-1]


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--sanitized" in sys.argv:
        print(build_sanitized())
