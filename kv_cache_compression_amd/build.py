"""Build libsnapkv.so in-tree with hipcc for gfx950.

    python -m kv_cache_compression_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["api.hip", "obs_score.hip", "obs_inst_bf16_d128.hip", "obs_inst_bf16_d64.hip", "obs_inst_f32_d128.hip",
           "obs_inst_f32_d64.hip", "obs_stream.hip", "obs_onepass.hip", "obs_onepass2.hip",
           "select_gather.hip", "select_split.hip", "decode.hip"]
LIB = os.path.join(PKG, "libsnapkv.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsnapkv)")


# Host-side sanitizers for the plan and validation code in api.hip (a test build; each flag goes
# to the host pass only, the device code is built as usual).
HOST_SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _compile(src: str, obj: str, extra=()) -> str:
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra) + ["-c", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                                                   os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
    return err


def build(verbose: bool = False, jobs: int = 0, out: str | None = None, host_sanitize: bool = False) -> str:
    """Compile every HIP source into kv_cache_compression_amd/libsnapkv.so (always rebuilds).
    The sources compile in parallel (one hipcc per source), then link into one library.
    out / host_sanitize: a test build elsewhere whose api.hip host code carries AddressSanitizer and
    UndefinedBehaviorSanitizer checks (load it with the sanitizer runtime preloaded)."""
    from concurrent.futures import ThreadPoolExecutor
    lib = out or LIB
    tag = "%d%s" % (os.getpid(), "s" if host_sanitize else "")
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + "." + tag + ".o") for s in SOURCES]
    extras = [HOST_SANITIZE_FLAGS if (host_sanitize and s == "api.hip") else [] for s in SOURCES]
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    try:
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            msgs = list(ex.map(_compile, SOURCES, objs, extras))
        tmp = lib + ".tmp" + tag
        res = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp],
                             capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    if verbose:
        for m in msgs:
            if m.strip():
                print(m, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
