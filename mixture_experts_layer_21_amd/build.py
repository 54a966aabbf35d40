"""Build the gfx950 MoE library (libmoe.so) in-tree with hipcc.

    python mixture_experts_layer_21_amd/build.py

(Run it by path: importing the package itself loads the library.)

Each HIP source compiles to an object under _build/, then one shared library
is linked next to this file.  It always recompiles (the build is the check
that the sources compile for gfx950).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["moe_api.hip", "route.hip", "permute.hip", "gemm_bf16.hip", "gemm_f32.hip",
           "combine.hip", "backward.hip", "noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the MoE library)")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 instructions stay off: plain fp32 code only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wall", "-Wno-unused-function",
    ]


# Host-side AddressSanitizer flavour (the device code is built as usual):
# every -fsanitize flag sits right after -Xarch_host, so it reaches only the
# host compilation of each source.
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, asan: bool = False) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".asan.o" if asan else ".o"))
    cmd = [hipcc(), *flags(), *(ASAN_FLAGS if asan else []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


ASAN_LIB = os.path.join(BUILD, "libmoe_asan.so")


def build(verbose: bool = True, asan: bool = False) -> str:
    """Build libmoe.so next to this file, or (asan) the host-sanitizer flavour
    _build/libmoe_asan.so, which a process loads with the sanitizer runtime
    preloaded (see tests/test_abi_asan.py)."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, asan), SOURCES))
    out = ASAN_LIB if asan else LIB
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC",
           *(["-Xarch_host", "-fsanitize=address", "-shared-libasan"] if asan else []), *objs,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(asan="--asan" in sys.argv[1:])
