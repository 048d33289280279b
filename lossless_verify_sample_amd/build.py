"""Build libssd.so (HIP, gfx950) in-tree with hipcc.

python -m lossless_verify_sample_amd.build [--phases]

--phases builds the instrumented libssd_phases.so instead (phase stamps of
the latency-bound kernels, read with ssd_phase_read; a measurement aid).
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "ssd.hip")
OUT = os.path.join(HERE, "libssd.so")
OUT_PHASES = os.path.join(HERE, "libssd_phases.so")
ARCH = os.environ.get("SSD_OFFLOAD_ARCH", "gfx950")


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def command(out, phases=False):
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        *(["-DSSD_PHASES"] if phases else []),
        # no FMA contraction: the host fan-out and the device offset bookkeeping
        # rely on plain IEEE operations; fused multiply-adds are written out
        "-ffp-contract=off",
        # packed fp32 ops (v_pk_*_f32) are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-o", out, SRC,
    ]


def build(verbose=True, phases=False):
    out = OUT_PHASES if phases else OUT
    tmp = out + ".tmp"
    cmd = command(tmp, phases)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msg)
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(phases="--phases" in sys.argv[1:])
    sys.exit(0)
