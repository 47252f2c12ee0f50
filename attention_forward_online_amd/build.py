"""Build libfa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m attention_forward_online_amd.build   (or build() from Python)

Every source is compiled for gfx950 only.  Packed fp32 VALU instructions are
disabled for device code (-packed-fp32-ops off); hipcc's host pass does not
know that target feature and says so, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libfa.so")
OBJ_DIR = os.path.join(PKG, "_build")

SOURCES = ["fa_api.hip", "fa_fwd_bf16.hip", "fa_fwd_f32.hip", "fa_decode.hip", "fa_softmax.hip", "fa_bwd_bf16.hip", "fa_bwd_f32.hip", "fa_fwd_v1.hip", "fa_probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source extra flags.  The bf16 prefill kernel is compiled assuming no NaN
# values (its masking works with -inf only; NaN inputs give unspecified
# output), which lets its row max skip quieting each matrix-core result.
FILE_FLAGS = {"fa_fwd_bf16.hip": ["-fno-honor-nans"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str, obj: str, hipcc: str) -> None:
    cmd = [hipcc, *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l and "(ignoring feature)" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if err.strip():
        print(err, file=sys.stderr)


def build(out_path: str = LIB_PATH, jobs: int = 4) -> str:
    """Compile every kernel source for gfx950 and link the shared library."""
    hipcc = _hipcc()
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, s.replace(".hip", ".o")) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], hipcc), zip(SOURCES, objs)))
    tmp = out_path + ".tmp"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build())
