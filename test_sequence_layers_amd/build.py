"""Build libttt.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

    python -m test_sequence_layers_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libttt.so")
SOURCES = ["abi.hip", "fullbatch.hip", "chunked.hip", "mlp.hip", "dwconv.hip", "grid.hip", "epilogue.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 ops are disabled for all device code: hipcc would otherwise form v_pk_* fp32
# instructions from ordinary float code.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]
# Per-source additions. MFMA accumulators in ordinary VGPRs: otherwise the compiler parks them in
# AGPRs and moves them back and forth (v_accvgpr_read/write) around every conversion of a result.
# Measured: causal TTT-Linear 91 -> 86 us; the TTT-MLP kernel (no AGPR moves either way) is left
# as it was. The chunk-step kernels (chunked scans, TTT-MLP) are chains of dependent short
# operations; the scheduler's ILP-maximising strategy orders them slightly better (bidirectional
# 46.1 -> 45.1 us, TTT-MLP 958 -> 947-954 us; the full-batch kernels are unchanged by it). For the
# split TTT-MLP schedule: 0.815-0.819 ms, against 0.826 (default), 0.828 (max-memory-clause), 0.840
# (iterative-ilp) and 0.858 ms (iterative-minreg).
SCHED_ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
SOURCE_FLAGS = {
    "fullbatch.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "chunked.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", *SCHED_ILP],
    "mlp.hip": SCHED_ILP,
}


def flags_for(src: str) -> list:
    return FLAGS + SOURCE_FLAGS.get(src, [])


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that noise.
    lines = [ln for ln in p.stdout.splitlines() if "packed-fp32-ops" not in ln]
    return p.returncode, "\n".join(lines)


def build(verbose: bool = False) -> str:
    """Compile every source and link libttt.so; returns its path. Raises on failure."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [HIPCC, *flags_for(src), "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    objs = []
    for src, obj, p in procs:
        out, _ = p.communicate()
        out = "\n".join(ln for ln in out.splitlines() if "packed-fp32-ops" not in ln)
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        raise RuntimeError(f"link failed:\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
