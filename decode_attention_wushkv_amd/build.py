"""Build libwushkv.so in-tree with hipcc for gfx950 (MI355X)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libwushkv.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("api.cpp", "append.hip", "decode.hip", "prefill.hip", "chunk.hip", "probe.hip", "noalloc.hip")]
HEADERS = [os.path.join(HERE, "csrc", h) for h in ("common.h", "quant.h", "chunk.h", "i8ops.h")] + [
    os.path.join(ROOT, "include", "wushkv.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # never emit packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source additions.  The chunked-step kernel keeps its int8 MFMA
# accumulators in VGPRs (no AGPR copies in its VALU-bound loop).
EXTRA_FLAGS = {"chunk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False) -> str:
    """Compile every source to an object (each with its flags) and link the
    shared library; the objects live in a temporary directory."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory() as td:
        def compile_one(src):
            obj = os.path.join(td, os.path.basename(src) + ".o")
            cmd = [hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
            return obj, subprocess.run(cmd, capture_output=True, text=True)

        with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
            results = list(ex.map(compile_one, SOURCES))
        for src, (obj, res) in zip(SOURCES, results):
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n" + res.stdout + res.stderr)
            if verbose:
                print(res.stderr)
        objs = [obj for obj, _ in results]
        res = subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                             capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
