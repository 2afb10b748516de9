"""Compile the FlashSampling HIP library (libflashsampling.so) for gfx950, in-tree."""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("fs_api.hip", "fs_kernels.hip", "fs_stream_flat.hip",
                                           "fs_stream_group.hip", "fs_stream_store.hip",
                                           "fs_stream_topk.hip")]
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libflashsampling.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    # packed fp32 vector ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libflashsampling.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _check(proc, what):
    out, err = proc.communicate()
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in err.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {what} ({proc.returncode}):\n{err}")


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the shared library."""
    os.makedirs(OBJDIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, os.path.basename(src).replace(".hip", ".o"))
        objs.append(obj)
        procs.append((_run([hipcc(), *HIPCC_FLAGS, *inc, "-c", src, "-o", obj], verbose), src))
    for proc, src in procs:
        _check(proc, src)
    tmp = LIB + ".tmp"
    _check(_run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose), "link")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
