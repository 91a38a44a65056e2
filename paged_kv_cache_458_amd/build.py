"""Build libpagedattn.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_458_amd.build
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libpagedattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed fp32 (v_pk_*_f32) instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def sources():
    """HIP sources (device and host code) and C++ sources (host code only)."""
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")) + glob.glob(os.path.join(PKG, "csrc", "*.cpp")))


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel, under _build/), then link one shared library; always
    rebuilds."""
    from concurrent.futures import ThreadPoolExecutor

    obj_dir = os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(obj_dir, os.path.basename(s) + ".o") for s in srcs]
    compile_flags = [f for f in FLAGS if f != "-shared"]

    def compile_one(so):
        src, obj = so
        cmd = [HIPCC, *compile_flags, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        return subprocess.run(cmd).returncode

    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(jobs) as ex:
        codes = list(ex.map(compile_one, zip(srcs, objs)))
    if any(codes):
        raise RuntimeError(f"hipcc failed for {[s for s, c in zip(srcs, codes) if c]}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def device_asm(out_dir: str) -> list[str]:
    """Write the gfx950 assembly of each source to out_dir (for inspecting instruction selection)."""
    os.makedirs(out_dir, exist_ok=True)
    outs = []
    for src in sources():
        if not src.endswith(".hip"):
            continue
        out = os.path.join(out_dir, os.path.basename(src).replace(".hip", ".s"))
        flags = [f for f in FLAGS if f not in ("-shared",)]
        subprocess.run([HIPCC, *flags, "-I", os.path.join(ROOT, "include"), "-S", "--cuda-device-only", src, "-o",
                        out], check=True)
        outs.append(out)
    return outs


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
