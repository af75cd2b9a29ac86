"""The C ABI used from plain C: tests/c_abi/abi_smoke.c is compiled with the
host C compiler against include/sparstar.h and linked to libsparstar.so (on
the CPU), and run on the GPU."""
import os
import subprocess
import shutil

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "abi_smoke.c")
LIBDIR = os.path.join(ROOT, "block_sparse_attention_head_amd")


def _build(out):
    cc = shutil.which("gcc") or shutil.which("cc")
    assert cc, "no C compiler"
    cmd = [cc, "-O1", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", SRC, "-o", out,
           "-L", LIBDIR, "-lsparstar", "-L", "/opt/rocm/lib", "-lamdhip64", "-lm",
           f"-Wl,-rpath,{LIBDIR}", "-Wl,-rpath,/opt/rocm/lib"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)


def test_c_program_compiles_and_links(tmp_path):
    out = str(tmp_path / "abi_smoke")
    _build(out)
    assert os.path.exists(out)


@pytest.mark.gpu
def test_c_program_runs(tmp_path):
    out = str(tmp_path / "abi_smoke")
    _build(out)
    r = subprocess.run([out], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_smoke ok" in r.stdout
