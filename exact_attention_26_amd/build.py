"""Build libfa.so (gfx950) in-tree with hipcc.

    python -m exact_attention_26_amd.build          # or __graft_entry__.build()

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled; the objects are linked into
exact_attention_26_amd/libfa.so next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["fa_fwd.hip", "fa_fwd_bf16.hip", "fa_bwd.hip", "fa_prefill.hip", "fa_rope.hip",
           "fa_decode.hip", "fa_api.cpp"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + INCLUDE, "-I" + CSRC]


# Per-source extra flags.  The bf16 forward, the paged prefill / tree and the
# RoPE forward (all built on fwd_block) keep every MFMA accumulator in VGPRs: the whole working set
# fits in 256 VGPRs at two waves per SIMD, and the softmax reads the score
# accumulators with VALU instructions.
EXTRA = {"fa_fwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "fa_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "fa_rope.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


# The benchmark's HBM read-rate probe: its own library, not part of libfa.so.
PROBE_SOURCE = "read_probe.hip"


def build_probe(verbose: bool = True) -> str:
    """Build libfa_probe.so (the read-bandwidth probe bench.py reports as
    context for the HBM-bound kernels)."""
    os.makedirs(BUILD, exist_ok=True)
    obj = _compile(PROBE_SOURCE)
    out = os.path.join(HERE, "libfa_probe.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out + ".tmp",
                        obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(out + ".tmp", out)
    if verbose:
        print(f"built {out}")
    return out


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    out = os.path.join(HERE, "libfa.so")
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    # a kernel whose host-side handle was not emitted shows up as an undefined
    # symbol of this library's own (anonymous-namespace) code: refuse it
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if "_GLOBAL__N_" in l]
    if nm.returncode == 0 and missing:
        raise RuntimeError(f"kernel handles missing from libfa.so: {missing}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build()
    build_probe()
