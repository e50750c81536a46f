"""Compile librq.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

The library is built in-tree next to this file so that it travels with the
source tree.  Packed-FP32 instruction selection is disabled (the kernels rely
on plain FP32 VALU ops).  The decode kernel's launcher is compiled once per
(head_dim, reference kind, chain mode) from rq_decode_inst.hip, and all
objects compile in parallel.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librq.so")
SOURCES = ["rq_api.cpp", "rq_encode.hip", "rq_reconstruct.hip", "rq_decode.hip", "rq_probe.hip"]
# (reference kind, chain mode) pairs the library dispatches to: BF16 reference
# or INT2/INT4 anchor with independent references; chained references (every
# slot, or slot 0 alone) over a BF16 or INT4 root.
DECODE_KINDS = [(0, 0), (2, 0), (4, 0), (0, 1), (4, 1), (0, 2), (4, 2)]
HEAD_DIMS = [64, 128, 256]
ARCH = os.environ.get("RQ_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def units():
    """(source, object name, extra flags) of every object of the library."""
    out = [(src, src.replace(".", "_") + ".o", []) for src in SOURCES]
    for aq, chain in DECODE_KINDS:
        for d in HEAD_DIMS:
            out.append(("rq_decode_inst.hip", f"rq_decode_d{d}_aq{aq}_chain{chain}.o",
                        [f"-DRQ_INST_D={d}", f"-DRQ_INST_AQ={aq}", f"-DRQ_INST_CHAIN={chain}"]))
    return out


def _newest_header() -> float:
    """Newest of every header (csrc/*.hpp, include/*.h) and this script."""
    paths = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hpp", ".h"))]
    inc = os.path.join(ROOT, "include")
    paths += [os.path.join(inc, f) for f in os.listdir(inc)]
    paths.append(os.path.abspath(__file__))
    return max(os.path.getmtime(p) for p in paths)


def build(verbose: bool = False, jobs: int = 0, force: bool = True) -> str:
    """Compile every object and link librq.so.  force=False skips objects
    newer than their source, every header and this script (for development
    rebuilds); the default compiles everything."""
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-fno-gpu-rdc", "-munsafe-fp-atomics"]
    jobs = jobs or min(16, os.cpu_count() or 4)
    headers = 0.0 if force else _newest_header()
    todo, objs = [], []
    for src, name, extra in units():
        obj = os.path.join(objdir, name)
        objs.append(obj)
        if (not force and os.path.exists(obj)
                and os.path.getmtime(obj) > max(headers, os.path.getmtime(os.path.join(CSRC, src)))):
            continue
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        todo.append((name, [hipcc()] + common + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]))

    def run(item):
        name, cmd = item
        if verbose:
            print(" ".join(cmd), flush=True)
        p = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
        err = "\n".join(x for x in p.stderr.splitlines() if "packed-fp32-ops" not in x)
        return name, p.returncode, err

    failed = []
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        for name, rc, err in pool.map(run, todo):
            if rc != 0:
                failed.append(name)
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
    print(build(verbose="-v" in sys.argv, force="--incremental" not in sys.argv))
