"""Build libsscnn.so (hipcc, gfx950) in-tree.

    python -m spatially_sharded_cnn_amd.build [-v]

Every source in csrc/ is compiled for gfx950 only, with packed FP32 vector
instructions disabled (-packed-fp32-ops), and linked into
spatially_sharded_cnn_amd/lib/libsscnn.so.  Objects go to _build/ at the repo
root.
"""
from __future__ import annotations

import concurrent.futures
import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD_DIR = ROOT / "_build" / "sscnn"
LIB_DIR = PKG / "lib"
LIB_PATH = LIB_DIR / "libsscnn.so"
ARCH = "gfx950"


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return p


def sources():
    return sorted(list(CSRC.glob("*.hip")) + list(CSRC.glob("*.cpp")))


COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: pathlib.Path, verbose: bool) -> pathlib.Path:
    obj = BUILD_DIR / (src.name + ".o")
    lang = ["-x", "hip"] if src.suffix == ".hip" else ["-x", "hip"]
    cmd = [hipcc()] + lang + COMMON_FLAGS + ["-c", str(src), "-o", str(obj)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src.name}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        # hipcc's host pass does not know the packed-fp32 feature; drop that noise.
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
        if any(l.strip() for l in lines):
            print("\n".join(lines), file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int = 0) -> pathlib.Path:
    """Compile every source and link libsscnn.so; returns its path."""
    BUILD_DIR.mkdir(parents=True, exist_ok=True)
    LIB_DIR.mkdir(parents=True, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB_PATH.with_suffix(".so.tmp%d" % os.getpid())
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", str(tmp)] + [str(o) for o in objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
