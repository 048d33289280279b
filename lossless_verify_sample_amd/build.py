"""Build libssd.so (HIP, gfx950) in-tree with hipcc.

python -m lossless_verify_sample_amd.build
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "ssd.hip")
OUT = os.path.join(HERE, "libssd.so")
ARCH = os.environ.get("SSD_OFFLOAD_ARCH", "gfx950")


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def command(out):
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # no FMA contraction: the host fan-out and the device offset bookkeeping
        # rely on plain IEEE operations; fused multiply-adds are written out
        "-ffp-contract=off",
        # packed fp32 ops (v_pk_*_f32) are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-o", out, SRC,
    ]


def build(verbose=True):
    tmp = OUT + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msg)
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
