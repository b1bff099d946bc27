"""Build libspecache.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m decode_attention_bit_kivi_amd.build  [--jobs N] [--asan OUT]

Every .hip file under csrc/ is compiled to an object for gfx950 and linked
into decode_attention_bit_kivi_amd/libspecache.so.  Packed-FP32 VALU
instructions are disabled for all device code (-packed-fp32-ops).

--asan OUT builds a second copy with AddressSanitizer in the host code only (argument
checks, workspace carving, stream helpers; the device code is built as usual) into OUT,
for the host-side tests run with the sanitizer's runtime preloaded.
"""
from __future__ import annotations

import argparse
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
OUT = os.path.join(PKG, "libspecache.so")
BUILD_DIR = os.path.join(os.path.dirname(PKG), "_build")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libspecache)")
    return exe


# AddressSanitizer for the host code only: each sanitizer flag is scoped to the host pass
ASAN_HOST_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def asan_runtime() -> str:
    """The AddressSanitizer runtime of the ROCm compiler (to preload into a host process)."""
    found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/lib/llvm")
    return found[-1]


def _compile(src: str, build_dir: str = BUILD_DIR, defines=(), extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        # hipcc's host pass warns about the device-only target feature; keep other warnings visible
        lines = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if lines:
            print("\n".join(lines), file=sys.stderr)
    return obj


def build(jobs: int = 8, verbose: bool = True, out: str = OUT, build_dir: str = BUILD_DIR,
          defines=(), asan: bool = False) -> str:
    """Compile every csrc/*.hip and link `out`; `defines` are extra NAME=VALUE macros; `asan`
    instruments the host code with AddressSanitizer."""
    os.makedirs(build_dir, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    extra = ASAN_HOST_FLAGS if asan else ()
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(sources)))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, defines, extra), sources))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} from {len(sources)} sources")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--asan", metavar="OUT", help="also build a host-AddressSanitizer copy into OUT")
    args = ap.parse_args()
    if args.asan:
        build(args.jobs, out=args.asan, build_dir=os.path.join(BUILD_DIR, "asan"), asan=True)
    else:
        build(args.jobs)


if __name__ == "__main__":
    main()
