"""Build libmiconv.so in-tree with hipcc for gfx950 (no GPU needed to build).

    python -m convolution_forward_conv2d_amd.build [--verbose]
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmiconv.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["miconv.cpp", "conv_fwd_mfma.hip", "conv_fwd_halo.hip", "conv_fwd_halo_bf16.hip",
           "conv_fwd_direct.hip", "conv_bwd_data.hip", "conv_bwd_filter.hip",
           "pool_fwd.hip", "brgemm.hip", "conv_bwd_filter_halo.hip",
           "conv_bwd_filter_split.hip", "conv_bwd_data_phase.hip", "conv_fwd_rows.hip",
           "conv_bwd_data_subpixel.hip", "conv_bwd_filter_rows.hip", "conv_bwd_filter_cl.hip",
           "conv_bwd_data_taps.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # packed fp32 VALU ops are off: hipcc would otherwise form v_pk_* fp32 ops on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in proc.stderr.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
        objs = list(pool.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv)
    print(LIB)
