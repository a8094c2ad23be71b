"""Build libdsa.so (gfx950) in-tree with hipcc.

    python -m sparse_attention_topk_amd.build      # or build() from Python

Each HIP source is compiled to an object in parallel, then linked into
sparse_attention_topk_amd/libdsa.so next to this file.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdsa.so")
# the checked build: the same sources with -DDSA_DEBUG (metadata validation,
# output and workspace canaries around every call; see dsa_debug_faults)
OBJ_DEBUG = os.path.join(HERE, "_build_debug")
LIB_DEBUG = os.path.join(HERE, "libdsa_debug.so")
SOURCES = ["api.hip", "cache_write.hip", "indexer_score.hip", "indexer_prefill.hip",
           "topk.hip", "sparse_mla.hip", "prologue.hip", "debug.hip"]
ARCH = os.environ.get("DSA_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]
# per-source code generation options
EXTRA = {
    # the prefill score kernel keeps its MFMA accumulators in VGPRs, where
    # the ReLU-weighted head sum reads them without accumulator moves
    "indexer_prefill.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
    # the one-token-per-workgroup attention keeps its queries (the logits'
    # B operands) in accumulator registers and its MFMA accumulators in
    # VGPRs; in the default form the queries spill into copies around every
    # MFMA.  The file's other kernels measure the same either way.
    "sparse_mla.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
}


def _compile(src, debug=False):
    obj = os.path.join(OBJ_DEBUG if debug else OBJ, os.path.splitext(src)[0] + ".o")
    cmd = ([HIPCC] + CFLAGS + (["-DDSA_DEBUG"] if debug else []) + EXTRA.get(src, []) +
           ["-c", os.path.join(CSRC, src), "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd),
                                                            r.stderr))
    return obj, r.stderr


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)


def build(verbose=False, debug=True):
    """Build libdsa.so and (debug=True) the checked build libdsa_debug.so."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = [(src, False) for src in SOURCES]
    if debug:
        os.makedirs(OBJ_DEBUG, exist_ok=True)
        jobs += [(src, True) for src in SOURCES]
    with ThreadPoolExecutor(max_workers=8) as ex:
        results = list(ex.map(lambda j: _compile(*j), jobs))
    if verbose:
        for _, err in results:
            if err.strip():
                sys.stderr.write(err)
    n = len(SOURCES)
    _link([o for o, _ in results[:n]], LIB)
    if debug:
        _link([o for o, _ in results[n:]], LIB_DEBUG)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, debug="--release-only" not in sys.argv))
