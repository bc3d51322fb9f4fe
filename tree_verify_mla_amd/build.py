"""Build libddtree.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m tree_verify_mla_amd.build [--verbose]

Every source under csrc/ is compiled to an object in _build/ (in parallel),
then linked into tree_verify_mla_amd/libddtree.so.  Packed-fp32 instruction
selection is disabled for all device code.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = ROOT / "_build"
LIB = PKG / "libddtree.so"
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}",
          "-Wall", "-Wno-unused-result"]
DEVICE_ONLY = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=fast"]
# Per-source options.  The matrix-core attention kernel keeps its output
# accumulators in AGPRs through inline asm and needs the builtin (score) MFMAs
# in their VGPR-accumulator form, which the compiler would otherwise not pick
# in a kernel that uses AGPRs.
SOURCE_FLAGS = {"verify_attn_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: Path, verbose: bool) -> Path:
    obj = BUILD / (src.name + ".o")
    # every source (the .cpp host files too) goes through the HIP language mode
    cmd = [hipcc(), "-x", "hip", *COMMON, "-c", str(src), "-o", str(obj), *DEVICE_ONLY,
           *SOURCE_FLAGS.get(src.name, [])]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l and "unused-command-line-argument" not in l
                     and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"compile failed for {src.name}:\n{msgs}")
    if verbose and msgs:
        print(msgs, flush=True)
    return obj


def device_asm(src_name: str, out: Path) -> Path:
    """gfx950 assembly of one source, compiled with the library's options."""
    src = CSRC / src_name
    cmd = [hipcc(), "-x", "hip", *COMMON, "--cuda-device-only", "-S", str(src), "-o", str(out),
           *DEVICE_ONLY, *SOURCE_FLAGS.get(src_name, [])]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"assembly of {src_name} failed:\n{res.stdout}{res.stderr}")
    return out


def build(verbose: bool = False) -> Path:
    BUILD.mkdir(exist_ok=True)
    srcs = sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.cpp"))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args()
    try:
        build(a.verbose)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
