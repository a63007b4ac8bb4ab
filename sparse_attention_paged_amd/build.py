"""Build libsap.so (the HIP kernels plus the C ABI of include/sap.h) for gfx950.

Usage: python -m sparse_attention_paged_amd.build
Each translation unit is compiled with hipcc in parallel, then linked into
sparse_attention_paged_amd/libsap.so next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsap.so")
ARCH = "gfx950"

# No fast-math and no denormal flushing: the format decoders and the softmax
# rely on IEEE fp32 behaviour.  Packed fp32 VALU ops are disabled for every
# device compile.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def check_no_scratch(remarks: str) -> None:
    """The attention kernels that gather rows with LDS DMA (bf16 rows, and
    e4m3 rows in the one-pass kernel at head_dim 512) count their own in-flight gathers with
    s_waitcnt vmcnt(N); a compiler-generated scratch access would be one more
    vector memory operation in that count.  Refuse such a build."""
    name = None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            # attn_kernel<D, KV, OUT, NW>: KV == 0 is bf16 (mangled ...ILi<D>ELi0E...);
            # attn_d512_kernel counts its gathers for bf16 and e4m3 rows alike
            if re.search(r"attn_kernelILi\d+ELi0E", name) or "attn_d512_kernel" in name:
                raise RuntimeError(f"{name} uses scratch memory ({m.group(1)} bytes/lane); "
                                   "its gather wait counts would be wrong")


def build(verbose: bool = False, jobs: int = 8) -> str:
    cc = hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = os.path.join(ROOT, "_build", "obj")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [cc, *FLAGS, "-c", src, "-o", obj]
        guard = os.path.basename(src) in ("attn.hip", "attn_d512.hip")
        if guard:
            cmd.append("-Rpass-analysis=kernel-resource-usage")
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{r.stderr}")
        if guard:
            check_no_scratch(r.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
