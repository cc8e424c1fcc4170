"""Build libmuon_mi355x.so for gfx950 in-tree with hipcc.

Usage: python -m newton_schulz_ns5_amd.build  (or call build()).
Every HIP source is compiled for gfx950 only, with packed fp32 instructions
disabled, and linked into one shared library next to this file.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmuon_mi355x.so")
SOURCES = ["gemm_bf16.hip", "gemm_f32.hip", "elementwise.hip", "poly_small.hip", "update_gram128.hip",
           "muon_host.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-mcode-object-version=5", "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-source flags.  The fused update/Gram kernel keeps two sets of MFMA
# accumulators live; with the MFMA operands and results in ordinary VGPRs the
# compiler does not shuttle one set between register files every sub-tile.
EXTRA = {"update_gram128.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src):
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, err in results:
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-mcode-object-version=5", "-shared", "-fPIC", "-o", tmp,
           *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
