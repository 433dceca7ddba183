"""Compile the HIP library libtrt.so for gfx950, in-tree.

`python -m thread_register_tile_amd.build` (or build()) compiles the
translation units of csrc/ with hipcc in parallel (objects in _build/) and
links thread_register_tile_amd/libtrt.so.  Packed-fp32 instruction selection
is switched off for all device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["trt.hip", "kern_tiny.hip", "kern_64.hip", "kern_128.hip", "kern_256.hip",
           "kern_256f.hip", "kern_dma256_f16_ak.hip", "kern_dma256_f16_am.hip",
           "kern_dma256_bf16_ak.hip", "kern_dma256_bf16_am.hip", "kern_dma192_f16.hip",
           "kern_dma192_bf16.hip", "kern_dma128.hip", "kern_skinny.hip", "kern_reduce.hip", "kern_f32.hip",
           "kern_regtile.hip"]
# Per-file flags.  The binary32 kernels keep their accumulators in ordinary
# VGPRs: left to itself the compiler puts them in AGPRs and moves half of
# them through VGPRs every K step.
FILE_FLAGS = {"kern_f32.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
LIB = os.path.join(HERE, "libtrt.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    "-fconstexpr-steps=100000000",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning
    # is expected and harmless.
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}")
    if verbose and err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = False, extra=(), jobs: int = 0) -> str:
    """Compile every translation unit (in parallel) and link libtrt.so."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *compile_flags, *FILE_FLAGS.get(src, []), *extra, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or max(1, min(len(cmds), len(os.sched_getaffinity(0)), 16))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"],
         verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
