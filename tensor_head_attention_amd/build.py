"""Builds libtha.so in-tree: every csrc/*.hip compiled by hipcc for gfx950, then linked.

Run as `python -m tensor_head_attention_amd.build` or call build_library().
Object files go to tensor_head_attention_amd/_build/ (not committed).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtha.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops off: the compiler must not form v_pk_{add,mul,fma}_f32.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-file code-generation options.  The backward kernels are compiler-scheduled with several
# live accumulator sets; the VGPR form of MFMA keeps their results out of AGPRs, which otherwise
# cost a copy back for every element the softmax-gradient step touches.
FILE_FLAGS = {
    "attn_bwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def generate_sources() -> None:
    """Regenerate the hand-scheduled attention loops (attn_loop_d128*.inc) from their generators."""
    for gen in ("gen_attn_loop.py", "gen_attn_loop_wide.py"):
        r = subprocess.run([sys.executable, os.path.join(CSRC, gen)], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"{gen} failed:\n{r.stdout}{r.stderr}")


def build_library(jobs: int = 8) -> str:
    """Generate the asm loop, compile every HIP source and link libtha.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    generate_sources()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library())
