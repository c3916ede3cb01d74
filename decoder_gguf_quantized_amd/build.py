"""Compile libqdec.so (HIP, gfx950) in place.

    python -m decoder_gguf_quantized_amd.build

Translation units, compiled in parallel into _build/ and linked with hipcc:
csrc/qdec.hip (runtime, attention / sampling / misc kernels and the C ABI),
csrc/kern_<type>.hip (the GEMV and GEMM instantiations of one weight type
each) and csrc/gguf.cpp (host-only: GGUF files and architecture definitions).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SRC = os.path.join(CSRC, "qdec.hip")
KERNEL_TYPES = ("f32", "q4_0", "q8_0", "q4_k", "q6_k")
SRCS_HIP = [SRC] + [os.path.join(CSRC, f"kern_{t}.hip") for t in KERNEL_TYPES]
SRC_HOST = os.path.join(CSRC, "gguf.cpp")
BUILD = os.path.join(HERE, "_build")
OUT = os.path.join(HERE, "libqdec.so")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    # packed-FP32 VALU forms stay off (the compiler would otherwise emit them
    # from plain float code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def _noise(text):
    return [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, os.path.splitext(os.path.basename(f))[0] + ".o") for f in SRCS_HIP]
    jobs = [[hipcc()] + HIPCC_FLAGS + ["-c", "-o", o, f] for o, f in zip(objs, SRCS_HIP)]
    objs.append(os.path.join(BUILD, "gguf.o"))
    jobs.append([os.environ.get("CXX", "g++")] + HOST_FLAGS + ["-c", "-o", objs[-1], SRC_HOST])
    procs = []
    for cmd in jobs:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    errors = []
    for cmd, p in zip(jobs, procs):
        out, _ = p.communicate()
        if p.returncode != 0:
            errors.append(f"{cmd[0]} {cmd[-1]} failed:\n" + "\n".join(_noise(out)))
        elif verbose and _noise(out):
            print("\n".join(_noise(out)))
    if errors:
        raise RuntimeError("\n".join(errors))
    tmp = OUT + ".tmp"
    link = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    if verbose:
        print(" ".join(link), flush=True)
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + "\n".join(_noise(r.stdout + r.stderr)))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
