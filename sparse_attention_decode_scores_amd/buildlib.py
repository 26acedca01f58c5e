"""Builds libdsa.so (the HIP kernels and the C entry points) in-tree for gfx950."""
import concurrent.futures
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
SOURCES = ["score.hip", "select.hip", "api.hip"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
         # keep the compiler from forming packed fp32 instructions
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # leading scalar and pointer kernel arguments (up to eight, stopping at the
         # first structure) arrive in scalar registers at wave launch
         "-mllvm", "-amdgpu-kernarg-preload-count=8",
         # a one-lane LDS atomic (a wave claiming the next unit of its chunk) stays a
         # plain atomic whose result is waited for where it is used; the atomic
         # optimizer's wave-wide form waited for it at once, ahead of the products
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
         "-I", os.path.join(ROOT, "include")]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose=False):
    """Compile every source and link libdsa.so; returns its path."""
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src + ".o")
        cmd = [cc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, r.stderr))
        if verbose and r.stderr.strip():
            print(r.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
