"""Build libwitcert.so (HIP, gfx950) in-tree with hipcc.

    python -m certified_kv_cache_amd.build [--verbose]

The library is compiled with -ffp-contract=off (the write path must agree bit
for bit with a float32 replay; every intended fused multiply-add is an
explicit fmaf), with packed fp32 VALU instructions disabled, and with MFMA
accumulators in ordinary VGPRs (the decode's output accumulators are also
rescaled by VALU code; the AGPR form copied them on every page).
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["write_kv.hip", "decode.hip", "gate.hip"]
LIB = os.path.join(HERE, "libwitcert.so")
ARCH = os.environ.get("WITCERT_ARCH", "gfx950")


def hipcc():
    for cand in [os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")]:
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def command(out=LIB, extra=()):
    srcs = [os.path.join(HERE, "csrc", s) for s in SOURCES]
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", os.path.join(ROOT, "include"), *extra, "-o", out, *srcs]


def build(verbose=False, out=LIB, extra=()):
    cmd = command(out, extra)
    tmp = out + ".tmp"
    cmd[cmd.index("-o") + 1] = tmp
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
