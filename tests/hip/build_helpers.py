"""Build the tests' own HIP helper library (tests/hip/libf64sums.so) with the
library's compile flags.  Called by the repository's build entry point."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
HELPER_LIB = os.path.join(HERE, "libf64sums.so")


def build_helpers(verbose: bool = False) -> str:
    import sys
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from block_sparse_attention_head_amd.build import compile_flags, hipcc
    out_tmp = HELPER_LIB + ".tmp"
    cmd = [hipcc(), *compile_flags(), "-shared", os.path.join(HERE, "f64_sums.hip"), "-o", out_tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the test helper failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(out_tmp, HELPER_LIB)
    if verbose:
        print(f"built {HELPER_LIB}", file=sys.stderr)
    return HELPER_LIB


if __name__ == "__main__":
    build_helpers(verbose=True)
