"""Build libmisa.so (the HIP library) in-tree with hipcc for gfx950.

Usage: python -m sparse_attention_indexer_block_amd.build  [--jobs N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmisa.so")
PROBE_LIB = os.path.join(HERE, "libmisa_probe.so")  # benchmark's streaming-floor probe
SOURCES = ["route_kernels.hip", "route_fast.hip", "score_kernels.hip", "topk_kernels.hip", "api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    # keep the compiler from forming packed fp32 ops on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# per-source flags: the scoring kernels keep MFMA accumulators in VGPRs, so the
# fused epilogue reads them without a copy out of the accumulation registers
EXTRA = {"score_kernels.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    # the benchmark's streaming-floor probe: a library of its own
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *CFLAGS, "-shared", os.path.join(CSRC, "stream_probe.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return LIB


def build_host_asan(out_dir: str, jobs: int = 4) -> str:
    """The library with its host code (argument validation, workspace
    planning, dispatch) instrumented with AddressSanitizer, as
    libmisa_asan.so in out_dir; the device code is built as usual, without
    sanitizer. It serves the CPU tests of the C ABI's validation paths, which
    return before any launch. Load it with the sanitizer runtime preloaded
    (asan_runtime())."""
    os.makedirs(out_dir, exist_ok=True)
    flags = [*CFLAGS, "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]

    def one(src):
        obj = os.path.join(out_dir, src.replace(".hip", ".asan.o"))
        r = subprocess.run([HIPCC, *flags, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"host ASan build failed for {src}:\n{r.stdout}{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(one, SOURCES))
    out = os.path.join(out_dir, "libmisa_asan.so")
    # the sanitizer runtime is not linked into a shared library; it is preloaded
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host ASan link failed:\n{r.stdout}{r.stderr}")
    return out


def asan_runtime() -> str:
    """The compiler's AddressSanitizer runtime (to preload), or '' if absent."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if path and os.path.isabs(path) and os.path.exists(path) else ""


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    print(build(ap.parse_args().jobs))
