"""Build libgattn.so (the HIP library behind include/gattn.h) for gfx950 with hipcc.

Every source is compiled in-tree into global_paged_gqa_amd/libgattn.so. Packed
fp32 VALU instructions are disabled for all device code.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgattn.so")
SOURCES = ["gattn.cpp", "graphs.cpp", "decode.hip", "combine.hip", "prefill.hip", "append.hip", "noalloc.hip"]
# Per-source extra hipcc flags. Decode: MFMA accumulators in VGPRs. Its softmax rescales the
# O accumulators with vector multiplies; held in AGPRs, they were copied to VGPRs and back on
# every page (a quarter of a page's instructions at head_dim 512). The prefill kernels keep
# theirs in AGPRs, which leaves the VGPRs to operand prefetch.
EXTRA = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def compile_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libgattn.so; always recompiles."""
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") or src.endswith(".cpp") else []
        cmd = [cc, *compile_flags(), *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.PIPE)
        objs.append(obj)
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
