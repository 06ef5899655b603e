"""Build liblightning_la.so (gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "liblightning_la.so")
SOURCES = ["la_abi.hip", "la_decode.hip", "la_scan.hip", "la_prefill_f32.hip", "la_prefill_bf16.hip"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops (v_pk_fma_f32 and kin).
HIPFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = ["hipcc", *HIPFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(line for line in out.decode(errors="replace").splitlines()
                         if "packed-fp32-ops" not in line)
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(text + "\n")
        elif verbose and text.strip():
            print(text)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB_PATH + ".tmp"
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
