"""Build libisg.so for gfx950 with hipcc (in-tree, no JIT cache).

Every translation unit is compiled for gfx950 only; packed-fp32 instruction
selection is switched off (-packed-fp32-ops) for all device code, and the
selection / sampling unit is built without floating-point contraction because
its fp32 arithmetic decides integers.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libisg.so")

SOURCES = ["util.hip", "cluster.hip", "select.hip", "attention.hip", "unpermute.hip", "pq.hip"]
EXTRA = {"select.hip": ["-ffp-contract=off"], "pq.hip": ["-ffp-contract=off"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def common_flags():
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", HERE]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (device code is built as
# usual): each flag goes to the host compilation only.
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]
SAN_DIR = os.path.join(BUILD, "sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libisg.so")


def build(verbose: bool = False, jobs: int = 8, sanitize: bool = False) -> str:
    """Build libisg.so in the package, or (sanitize=True) the host-sanitized build
    _build/sanitize/libisg.so, which the sanitizer test loads through ISG_LIBRARY
    with the compiler's AddressSanitizer runtime preloaded."""
    bdir = SAN_DIR if sanitize else BUILD
    lib_out = SAN_LIB if sanitize else LIB
    os.makedirs(bdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        cmd = ([cc, "-c", os.path.join(HERE, src), "-o", obj] + common_flags() + EXTRA.get(src, []) +
               (SAN_HOST if sanitize else []))
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        if out.strip() and verbose:
            print(out, flush=True)
        return obj

    with ThreadPoolExecutor(max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = lib_out + ".tmp"
    cmd = [cc, "-shared", "--offload-arch=gfx950", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, lib_out)
    return lib_out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
