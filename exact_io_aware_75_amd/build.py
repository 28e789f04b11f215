"""Build libattn.so in-tree with hipcc for gfx950.

    python -m exact_io_aware_75_amd.build        # or __graft_entry__.build()

Each HIP source is compiled to an object under _build/ and linked into
exact_io_aware_75_amd/libattn.so (the attention library) or
exact_io_aware_75_amd/libattn_probe.so (the MFMA throughput probe).  Always recompiles (the build is the
"does it build" check).
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ("attn_api.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_std.hip")
# The MFMA throughput probe the benchmark measures its ceiling with: a
# separate library, not part of the attention ABI.
PROBE_SOURCES = ("mfma_probe.hip",)
# Per-file extra flags.  The forward kernel forms no NaN from finite inputs
# in any value it uses: masked scores are -inf, and where -inf could meet -inf
# or 0 (the scaled row max of a row with no key in a tile when scale = 0; the
# rescale factor, probability shift and final division of a row that has no
# key) it selects -inf, 1, 0 or 0 instead.  The one NaN left, a masked score
# times scale 0 inside exp2, is discarded by a select on the score.  So
# NaN-preserving max semantics are dropped there: v_max3 then needs no
# canonicalising v_max per MFMA result.  Host-side argument validation
# (attn_api.hip, which tests for NaN scales) keeps full IEEE semantics.
FILE_FLAGS = {"attn_fwd.hip": ["-fno-honor-nans"]}
LIB = os.path.join(HERE, "libattn.so")
PROBE_LIB = os.path.join(HERE, "libattn_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(srcs), 5)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s_] for s_ in SOURCES], LIB)
    _link([objs[s_] for s_ in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
