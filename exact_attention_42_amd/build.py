"""Build libattn.so (the C-ABI library with the gfx950 kernels) in place with hipcc.

Run ``python exact_attention_42_amd/build.py`` (a plain script: it does not import the package,
whose import loads the library being rebuilt) or call :func:`build`. The library is written
next to this file; the sources are ``csrc/*.hip`` and the public header ``include/attn.h``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
# The same library with every kernel's LDS filled with NaN bytes before use (-DATTN_POISON_LDS):
# a check build whose results must equal libattn.so's bit for bit. Only the tests load it.
LIB_POISON = os.path.join(PKG, "libattn_poison.so")
POISON_FLAGS = ("-DATTN_POISON_LDS",)
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU instructions.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source extras. The bf16 forward never relies on NaN semantics (masked scores are
# -inf, never NaN), and without NaN honouring each fmaxf on a matrix-core result no longer
# needs a canonicalising v_max first, which halves the row-max cost of the softmax.
FILE_FLAGS = {
    "attn_fwd_bf16.hip": ["-fno-honor-nans"],
    "attn_fwd_paged.hip": ["-fno-honor-nans"],
    # the decode kernel needs few registers; with the accumulators in ordinary VGPRs the
    # per-block rescale runs on them directly instead of copying through AGPRs
    "attn_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    # the wide forward: score accumulators must be ordinary VGPRs (the softmax reads them);
    # the register allocator then keeps the K/Q operands in the accumulation registers
    "attn_fwd_wide.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libattn.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout or "") + (r.stderr or "")
    # the host pass does not know the packed-fp32 feature name; that warning is expected
    lines = [l for l in out.splitlines() if "not a recognized feature for this target" not in l]
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    """Compile every csrc/*.hip for gfx950 and link libattn.so (or ``out``). Returns its path."""
    hipcc = _hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    objdir = os.path.join(PKG, "_build", hashlib.sha1(" ".join(extra_flags).encode()).hexdigest()[:8])
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    flags = HIPCC_FLAGS + list(extra_flags) + ["-I", INCLUDE, "-I", CSRC]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        futs = [ex.submit(_run, [hipcc] + flags + FILE_FLAGS.get(os.path.basename(s), [])
                          + ["-c", s, "-o", o], verbose)
                for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = out + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> None:
    """libattn.so, then the LDS-poisoning check build next to it."""
    build(verbose)
    build(verbose, extra_flags=POISON_FLAGS, out=LIB_POISON)


if __name__ == "__main__":
    build_all(verbose="-v" in sys.argv)
    print(LIB)
    print(LIB_POISON)
