"""The library used from plain C: tests/c/abi_check.c includes only the
public headers (include/*.h), is compiled by gcc as strict C99 and linked
against the built library, and checks sizes, layouts, status strings and the
host-side validation of every entry point (no call reaches the GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "mixture_experts_ffn_moe_amd")
SRC = os.path.join(ROOT, "tests", "c", "abi_check.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_c_program_against_the_headers(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libmoe_mi355x.so")):
        pytest.fail("libmoe_mi355x.so is not built (python __graft_entry__.py build)")
    exe = str(tmp_path / "abi_check")
    cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I",
                         os.path.join(ROOT, "include"), SRC, "-L", LIBDIR, "-lmoe_mi355x",
                         f"-Wl,-rpath,{LIBDIR}", "-o", exe], capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "abi_check ok" in run.stdout
