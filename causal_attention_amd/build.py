"""Build libcausal_attn.so in-tree with hipcc for gfx950.

    python -m causal_attention_amd.build

The library is written next to this file so that it travels with the source
tree; nothing is installed anywhere else.
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libcausal_attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["attn_api.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_bwd_doc.hip", "attn_decode.hip", "attn_rope.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-result",
    # matrix-core accumulators in VGPRs: the softmax reads them directly
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # keep the compiler from forming packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# Per-source flags.  The causal backward kernels are scheduled with the
# compiler's iterative ILP strategy: measured on MI355X (backward, bitwise
# equal results) ctx 1024 96.3 -> 93.4 us, ctx 512 37.6 -> 36.0, 4 K/V heads
# at S = 8192 1.47 -> 1.40 ms, packed documents 84.4 -> 85.8; on the forward
# it made no difference.  The packed-document instantiations
# (attn_bwd_doc.hip) keep the default strategy: with the work-ranked
# document schedule the iterative one crashes this compiler's register
# allocator on one of them, and it did not help packed documents before.
FILE_FLAGS = {
    "attn_bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}


def source_digest() -> str:
    """Digest of everything the library is built from: every file under csrc/,
    the public header and the compiler flags (global and per source).  The build embeds it in the
    library (attn_build_id), and the binding refuses a library whose digest
    differs from the tree's, so a stale build never runs in its place."""
    h = hashlib.sha256()
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))
    for name in files:
        h.update(name.encode() + b"\0")
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(INCLUDE, "attn_api.h"), "rb") as f:
        h.update(f.read())
    h.update(" ".join(HIPCC_FLAGS).encode())
    for name in sorted(FILE_FLAGS):
        h.update((name + ":" + " ".join(FILE_FLAGS[name])).encode())
    return h.hexdigest()[:16]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build the attention library")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (proc.stdout + proc.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile each source to an object (in parallel), then link the library."""
    from concurrent.futures import ThreadPoolExecutor
    import tempfile
    flags = [*HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", f"-I{CSRC}",
             f'-DATTN_SOURCE_DIGEST="{source_digest()}"']
    compile_flags = [f for f in flags if f != "-shared"]
    tmp = LIB_PATH + ".tmp"
    with tempfile.TemporaryDirectory(prefix="attn_build_") as objdir:
        objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[hipcc(), *compile_flags, *FILE_FLAGS.get(s, []), "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
