"""Build libwitcert.so (HIP, gfx950) in-tree with hipcc.

    python -m certified_kv_cache_amd.build [--verbose]
    python -m certified_kv_cache_amd.build --sanitized OUT.so   (host ASan/UBSan)

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


# Host code under AddressSanitizer and UndefinedBehaviorSanitizer (device
# code unoptimized and uninstrumented), for the argument checks and host
# glue on machines without a GPU.  The library expects the ASan runtime to be
# preloaded into the process (asan_runtime()).
SAN_FLAGS = ["-O1", "-g",
             "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xarch_device", "-O0", "-Xarch_device", "-g0"]


def asan_runtime():
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the clang ASan runtime was not found")
    return path


def build_sanitized(out):
    """Compile the sources in parallel with SAN_FLAGS and link `out`."""
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(os.path.dirname(out), src + ".o")
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-ffp-contract=off",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN_FLAGS,
               "-I", os.path.join(ROOT, "include"), "-c", "-o", obj, os.path.join(HERE, "csrc", src)]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    failed = [p.communicate()[0] for p in procs if p.wait() != 0]
    if failed:
        sys.stderr.write("\n".join(failed))
        raise RuntimeError("hipcc failed")
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-shared-libsan",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", out, *objs]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    return out


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        print(build_sanitized(sys.argv[sys.argv.index("--sanitized") + 1]))
    else:
        print(build(verbose="--verbose" in sys.argv))
