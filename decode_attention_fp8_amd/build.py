"""Build libpkv.so (the HIP kernels and the C ABI) for gfx950, in place.

    python decode_attention_fp8_amd/build.py

Compiles every source under csrc/ with hipcc (one object each, in parallel)
and links them into decode_attention_fp8_amd/libpkv.so. No fast-math; packed
FP32 instructions are disabled in the device code (-packed-fp32-ops). The
MFMA grouped-query kernel is built with MFMA results in ordinary VGPRs: its
32 accumulators then stay put across the token loop instead of being copied
between register files every tile.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpkv.so")
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")) +
                  glob.glob(os.path.join(HERE, "csrc", "*.cpp")))


# per-source device code generation options: MFMA results in VGPRs (with
# them in AGPRs the compiler copies the accumulators across the register
# files every tile: 80 copies per tile in the drafts kernel)
EXTRA = {"decode_gqa_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "decode_drafts.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def compile_command(src: str, obj: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            *EXTRA.get(os.path.basename(src), []),
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
            src, "-o", obj]


def link_command(objs: list[str], out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", *objs, "-o", out]


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with exit code {r.returncode}: {' '.join(cmd[-3:])}")


def build(verbose: bool = False) -> str:
    jobs = min(8, os.cpu_count() or 1)
    with tempfile.TemporaryDirectory(prefix="pkv_build_") as tmpdir:
        srcs = sources()
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            for f in [ex.submit(_run, compile_command(s, o), verbose) for s, o in zip(srcs, objs)]:
                f.result()
        tmp = LIB + ".tmp"
        _run(link_command(objs, tmp), verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
