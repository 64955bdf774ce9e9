"""Ahead-of-time build of the HIP library for gfx950.

``python -m varlen_attention_forward_amd.build`` compiles
``csrc/varlen_attn_fwd.hip``, ``csrc/varlen_attn_fwd_fp8.hip`` and
``csrc/merge_states.hip`` into
``libvarlen_attn.so`` next to this file.
hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
LIB_NAME = "libvarlen_attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = [
    os.path.join(CSRC, "varlen_attn_fwd.hip"),
    os.path.join(CSRC, "varlen_attn_fwd_fp8.hip"),
    os.path.join(CSRC, "varlen_attn_short.hip"),
    os.path.join(CSRC, "merge_states.hip"),
]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Inputs are finite and masked scores are -inf, never NaN: lets fmaxf map
    # to v_max3_f32 without NaN-quieting copies.
    "-fno-honor-nans",
    # MFMA results in VGPRs even where a wave has more than 256 registers
    # (one wave per SIMD): the softmax reads the score tiles with plain VALU
    # ops, which AGPR results would first have to be copied out for.
    "-mllvm",
    "-amdgpu-mfma-vgpr-form=1",
    # Keep the compiler from forming packed fp32 VALU ops in device code.
    "-Xclang",
    "-target-feature",
    "-Xclang",
    "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    return res.returncode, "\n".join(l for l in res.stderr.splitlines() if noise not in l)


def build(verbose: bool = False) -> str:
    """Compile the library in place and return its path.

    Each source is compiled to its own object in parallel (each carries its
    own gfx950 code object), then the objects are linked into one library."""
    from concurrent.futures import ThreadPoolExecutor
    import tempfile

    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    with tempfile.TemporaryDirectory(prefix="va_build_") as objdir:
        objs, cmds = [], []
        for src in SOURCES:
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            objs.append(obj)
            cmds.append([hipcc()] + HIPCC_FLAGS + ["-c", "-I", INCLUDE, "-I", CSRC, "-o", obj, src])
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            results = list(ex.map(_run, cmds))
        link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
        for rc, err in results:
            if rc != 0:
                raise RuntimeError("hipcc failed (%d):\n%s" % (rc, err))
            if verbose and err.strip():
                print(err, file=sys.stderr)
        if verbose:
            print(" ".join(link), flush=True)
        rc, err = _run(link)
        if rc != 0:
            if os.path.exists(tmp):
                os.remove(tmp)
            raise RuntimeError("hipcc link failed (%d):\n%s" % (rc, err))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
