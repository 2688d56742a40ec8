"""Build libsepattn.so (gfx950) in-tree with hipcc.

    python -m kv_cache_compression_sep_amd.build

Compiles every HIP source under csrc/ for gfx950 and links one shared
library next to this file. Packed-fp32 VALU instructions are disabled
(``-packed-fp32-ops``); hipcc's host pass warns that it does not know the
feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsepattn.so")
SOURCES = ["api.hip", "mask.hip", "compact.hip", "prefill.hip", "prefill_bf16.hip", "prefill_bwd.hip",
           "prefill_bwd_bf16.hip", "cache.hip", "decode.hip", "chunk.hip", "noalloc.hip"]
# Per-source code generation: the bf16 backward kernels keep their MFMA
# accumulators in VGPRs (with AGPRs as the accumulators the compiler copies
# them between the two files every tile).
EXTRA_FLAGS = {"prefill_bwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = os.environ.get("SEPATTN_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # the LDS-DMA asm statements name M0 (reserved) as clobbered on purpose
    "-Wno-inline-asm",
    # no kernel tests for NaN; without this every fmaxf also canonicalises
    "-fno-honor-nans",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 6) -> str:
    hipcc = _hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [hipcc, *FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            noise = "is not a recognized feature for this target"
            msg = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
            if msg.strip():
                print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
