"""Build libmtd.so (HIP kernels for gfx950 + the C-ABI host layer) in-tree with hipcc.

    python -m gqa_kv_cache_qwen3_amd.build        # or gqa_kv_cache_qwen3_amd.build.build()

Every source is compiled for gfx950 only.  Packed fp32 VALU instructions are disabled for device
code; the host pass ignores that feature with a harmless warning.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmtd.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["mtd_api.cpp", "kv_append.hip", "decode.hip", "prefill.hip", "proj.hip", "merge.hip", "measure.hip"]
# Per-file flags.  The prefill kernel never sees a NaN score (keys past a request's end are read
# from a valid row of its page), so its maxima need no NaN canonicalisation.
FILE_FLAGS = {"prefill.hip": ["-fno-honor-nans"]}

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON_FLAGS = [
    "--offload-arch=gfx950",
    "-mcode-object-version=5",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON_FLAGS, *FILE_FLAGS.get(src, []), *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr).strip()
    # the host pass does not know the device-only target feature; keep the log quiet about it
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    out = "\n".join(line for line in out.splitlines() if line.strip() != noise)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{out}")
    if out:
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = True, extra_flags: list[str] | None = None) -> str:
    """Compile every source and link libmtd.so next to this file.  Returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra_flags or [])
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build()
