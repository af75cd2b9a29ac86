"""Compile the HIP sources into the in-tree shared library ``libsparstar.so``.

Run ``python -m block_sparse_attention_head_amd.build`` (or call ``build()``).
Every source is compiled for gfx950 only; object files are built in parallel
and linked with hipcc.  hipcc's host pass warns that it does not know the
``packed-fp32-ops`` target feature; that warning is expected.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsparstar.so")
SOURCES = ["api.hip", "block_means.hip", "block_scores.hip", "select_blocks.hip",
           "screen_select.hip", "attn_fwd_bf16.hip", "attn_fwd_f32.hip", "retained_mass.hip",
           "transfer_scores.hip", "token_bound.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the SparSTAR HIP library cannot be built")


def compile_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-I", os.path.join(ROOT, "include"),
            # packed fp32 VALU ops stay off for all device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-result"]


def build(verbose: bool = False, jobs: int = 6) -> str:
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="sparstar_build_")
    try:
        def one(src):
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            msg = "\n".join(x for x in (r.stdout + r.stderr).splitlines()
                            if "packed-fp32-ops" not in x)
            if r.returncode != 0:
                raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{msg}")
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
            return obj

        with ThreadPoolExecutor(max_workers=jobs) as ex:
            objs = list(ex.map(one, SOURCES))
        out_tmp = LIB + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", out_tmp,
               *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
        os.replace(out_tmp, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
