"""Compile librq.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

The library is built in-tree next to this file so that it travels with the
source tree.  Packed-FP32 instruction selection is disabled (the kernels rely
on plain FP32 VALU ops).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librq.so")
SOURCES = ["rq_api.cpp", "rq_encode.hip", "rq_reconstruct.hip", "rq_decode.hip",
           "rq_decode_anchor4.hip", "rq_decode_anchor2.hip", "rq_decode_chain0.hip",
           "rq_decode_chain4.hip", "rq_decode_chain0_one.hip", "rq_decode_chain4_one.hip"]
ARCH = os.environ.get("RQ_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, jobs: int = 4) -> str:
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-fno-gpu-rdc", "-munsafe-fp-atomics"]
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".", "_") + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [hipcc()] + common + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        _, err = p.communicate()
        err = "\n".join(x for x in err.splitlines() if "packed-fp32-ops" not in x)
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(err + "\n")
        elif verbose and err.strip():
            sys.stderr.write(err + "\n")
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    link = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,--no-undefined", "-o",
            LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
