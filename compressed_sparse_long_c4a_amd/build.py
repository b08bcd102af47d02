"""Build libcsa.so (the HIP kernels and their C ABI) in-tree for gfx950 with hipcc."""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libcsa.so")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    "--offload-arch=gfx950",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# Per-source extra hipcc flags: MFMA accumulators in ordinary VGPRs.  index.hip: the score
# epilogue (relu, head weights) reads them without one v_accvgpr_read per value.  attn.hip: the
# one-wave-per-SIMD bf16 kernel scales its output accumulators in place when the softmax
# reference moves (with them in AGPRs every value is copied out and back, and the copies of
# all 144 at once made the register allocator spill); the other attention kernels run at two
# waves per SIMD and use no AGPRs either way.
FILE_FLAGS: dict[str, list[str]] = {"index.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                                    "attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcsa)")


def build(verbose: bool = False, src_dir: str | None = None, out: str | None = None,
          extra_flags: list[str] | None = None, link_flags: list[str] | None = None) -> str:
    """Compile every .hip source of csrc/ (or src_dir) and link one shared library (LIB or out).
    extra_flags / link_flags: additional hipcc options for every compile / for the link."""
    src_dir = src_dir or os.path.join(PKG, "csrc")
    out = out or LIB
    srcs = sorted(glob.glob(os.path.join(src_dir, "*.hip")))
    inc = ["-I", os.path.join(ROOT, "include"), "-I", src_dir]
    with tempfile.TemporaryDirectory(prefix="csa_build_") as tmpdir:
        def compile_one(src: str) -> str:
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *(extra_flags or []),
                   *inc, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            return obj

        with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            objs = list(ex.map(compile_one, srcs))
        tmp = out + ".tmp"
        cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *(link_flags or []), *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
