"""Build libmla.so (HIP for gfx950) in-tree with hipcc.

Usage: python mla_latent_kv_39_amd/build_lib.py   (or __graft_entry__.build()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla.so")
SOURCES = ["mla_api.cpp", "mla_decode_asm.cpp", "mla_combine.hip", "mla_check.hip", "mla_noalloc.hip",
           "mla_proj.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla)")


def flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # packed fp32 VALU forms stay off: the compiler emits ordinary fp32 code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include")]


LLVM_BIN = "/opt/rocm/lib/llvm/bin"


def build_asm_kernel(objdir: str, verbose: bool = False) -> str:
    """Generate the decode kernel's assembly, assemble and link it into a code
    object, and wrap its bytes in a C++ source; returns that source's path."""
    asm = os.path.join(objdir, "mla_decode_gfx950.s")
    obj = os.path.join(objdir, "mla_decode_gfx950.o")
    co = os.path.join(objdir, "mla_decode_gfx950.co")
    cpp = os.path.join(objdir, "mla_decode_gfx950_co.cpp")
    steps = [[sys.executable, os.path.join(CSRC, "gen_decode_gfx950.py"), asm],
             [os.path.join(LLVM_BIN, "clang"), "-x", "assembler", "-target", "amdgcn-amd-amdhsa",
              f"-mcpu={ARCH}", "-c", asm, "-o", obj],
             [os.path.join(LLVM_BIN, "ld.lld"), "-shared", obj, "-o", co]]
    for cmd in steps:
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"{cmd[0]} failed:\n{res.stderr}")
    data = open(co, "rb").read()
    body = ",".join(str(b) for b in data)
    with open(cpp, "w") as f:
        f.write("// generated from mla_decode_gfx950.co by build_lib.py\n")
        f.write(f'extern "C" const unsigned char mla_decode_gfx950_co[{len(data)}] '
                f'__attribute__((aligned(4096))) = {{{body}}};\n')
        f.write(f'extern "C" const unsigned long mla_decode_gfx950_co_size = {len(data)};\n')
    return cpp


def build(verbose: bool = False) -> str:
    """Compile every source and link libmla.so next to this file; returns its path."""
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    co_cpp = build_asm_kernel(objdir, verbose)
    obj = os.path.join(objdir, "mla_decode_gfx950_co.o")
    res = subprocess.run(["g++", "-O1", "-fPIC", "-c", co_cpp, "-o", obj], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling the embedded code object failed:\n{res.stderr}")
    objs.append(obj)
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
