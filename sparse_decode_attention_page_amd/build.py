"""Build libentmaxkv.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m sparse_decode_attention_page_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libentmaxkv.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["abi.hip", "meta.hip", "score.hip", "topk.hip", "gauss.hip", "group.hip", "decode.hip", "decode_items.hip", "softmax.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",                       # fused multiply-adds only where written
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Wno-unused-result",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build_host_sanitized(out: str, jobs: int | None = None) -> str:
    """The library with its host code (argument validation, workspace sizing,
    launch set-up) under AddressSanitizer and UndefinedBehaviorSanitizer (the
    GPU code is built as usual, without them) into `out`: for CPU runs of the
    checks that fail before any launch, in a process started with clang's ASan
    runtime preloaded.  Skipped when `out` is newer than every source."""
    srcs = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(ROOT, "include", "entmaxkv.h")]
    if os.path.exists(out) and os.path.getmtime(out) > max(os.path.getmtime(f) for f in srcs):
        return out
    tmp = out + ".objs"
    os.makedirs(tmp, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

    def comp(src: str) -> str:
        obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
        cmd = ["hipcc", *FLAGS, "-Xarch_host", "-g", *san, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(jobs or min(len(SOURCES), os.cpu_count() or 4, 8)) as ex:
        objs = list(ex.map(comp, SOURCES))
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *san, "-o", out, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return out


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    subprocess.check_call(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else None))
