"""Compile libqdec.so (HIP, gfx950) in place.

    python -m decoder_gguf_quantized_amd.build
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "qdec.hip")
OUT = os.path.join(HERE, "libqdec.so")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # packed-FP32 VALU forms stay off (the compiler would otherwise emit them
    # from plain float code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def build(verbose=False):
    tmp = OUT + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + ["-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
