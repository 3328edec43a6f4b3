"""Build librar.so (the HIP C-ABI library) for gfx950 with hipcc, in tree.

Each .hip source is compiled to an object in parallel, then linked into
ring_all_reduce_scatter_amd/librar.so.  Flags:
  -ffp-contract=off                   no FMA contraction: sums stay plain adds
  -fno-gpu-flush-denormals-to-zero    binary32 subnormals are kept
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                      no packed-fp32 instructions are generated
"""
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librar.so")

ARCH = os.environ.get("RAR_OFFLOAD_ARCH", "gfx950")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _filter(stderr: str) -> str:
    # the host pass does not know the packed-fp32 target feature; that note is harmless
    keep = [ln for ln in stderr.splitlines() if "packed-fp32-ops" not in ln]
    return "\n".join(keep)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    procs = []
    objs = []
    for src in srcs:
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        cmd = [cc, *CFLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, err = p.communicate()
        msg = _filter(err)
        if msg.strip() and (verbose or p.returncode):
            print(msg, file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    if r.returncode:
        print(_filter(r.stderr), file=sys.stderr)
        raise RuntimeError("link of librar.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
