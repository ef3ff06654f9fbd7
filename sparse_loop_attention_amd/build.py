"""Builds libflashloop.so (all HIP sources, gfx950) in-tree with hipcc.

Usage: python -m sparse_loop_attention_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libflashloop.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["api.hip", "timing.hip", "select.hip", "kv.hip", "attn_rows.hip", "attn_decode.hip", "attn_plan.hip", "attn_mfma.hip", "scratch.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions anywhere in the library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# host code (argument validation, planning, launches) under AddressSanitizer
# and UndefinedBehaviorSanitizer, for the CPU tests of the C ABI; device code
# is built as usual.  The library then needs the sanitizer runtime preloaded.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
SANITIZED_OUT = os.path.join(BUILD, "asan", "libflashloop.so")


def sanitizer_runtime() -> str:
    """The sanitizer runtime that a sanitized library needs preloaded."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD, "asan" if sanitize else "", src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *(SANITIZE if sanitize else []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 8, sanitize: bool = False) -> str:
    """Builds libflashloop.so in the package (sanitize: _build/asan/libflashloop.so)."""
    out = SANITIZED_OUT if sanitize else OUT
    os.makedirs(os.path.dirname(out) if sanitize else BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)
    return out


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--sanitize", action="store_true", help="host code under ASan + UBSan (CPU tests)")
    args = ap.parse_args()
    print(build(args.jobs, args.sanitize))


if __name__ == "__main__":
    main()
