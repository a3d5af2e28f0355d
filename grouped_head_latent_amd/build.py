"""Build libgha.so (the C-ABI library and its gfx950 kernels) in-tree with hipcc.

    python -m grouped_head_latent_amd.build

Every HIP source is compiled for gfx950 only.  Packed-fp32 VALU instructions
are disabled in device code (-packed-fp32-ops); the host pass warns that it
does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libgha.so")
OBJDIR = os.path.join(ROOT, "_build", "gha")
SOURCES = ["abi.cpp", "prefill_bf16.hip", "prefill_d128.hip", "prefill_f32.hip", "gta.hip", "decode.hip",
           "stream_decode.hip", "latent.hip", "absorb.hip", "noalloc.hip", "gta_fused.hip", "checks.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wno-unused-result"]


# Per-source flags.  The d = 128 prefill, GTA and streaming decode kernels
# never see NaN scores (rows past the sequence end read as zeros and masked
# scores are -inf), so fmaxf there needs no NaN canonicalisation of its
# operands.
SOURCE_FLAGS = {"prefill_d128.hip": ["-fno-honor-nans"], "gta.hip": ["-fno-honor-nans"],
                "gta_fused.hip": ["-fno-honor-nans"],
                "stream_decode.hip": ["-fno-honor-nans"]}


def _compile(src: str, extra=(), objdir=None) -> str:
    objdir = objdir or OBJDIR
    os.makedirs(objdir, exist_ok=True)
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *SOURCE_FLAGS.get(src, []), *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, save_temps: bool = False, defines=(), out: str | None = None) -> str:
    """Compile every source and link libgha.so (or `out`); returns its path.
    `defines` are extra -D tuning knobs."""
    extra = ["-save-temps=obj"] if save_temps else []
    extra += [f"-D{d}" for d in defines]
    target = out or LIB
    objdir = OBJDIR if out is None else os.path.join(OBJDIR, os.path.basename(out) + ".objs")
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, objdir), SOURCES))
    tmp = target + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, target)
    if verbose:
        print(f"built {target}")
    return target


def clean() -> None:
    shutil.rmtree(OBJDIR, ignore_errors=True)


if __name__ == "__main__":
    build(verbose=True, save_temps="--save-temps" in sys.argv)
