"""The C ABI from plain C: tests/c_abi_check.c includes include/jscan.h under
-std=c99 -Wall -Wextra -pedantic -Werror, links against the built
libjscan.so, resolves every entry point and calls the ones that do no GPU
work (sizes, plan, status strings, argument rejection).  CPU only."""
import os
import shutil
import subprocess

import pytest

import selective_state_space_11_amd as js

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_header_compiles_and_links_from_c(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(js.LIB_PATH):
        from selective_state_space_11_amd import build
        build.build()
    exe = tmp_path / "c_abi_check"
    libdir = os.path.dirname(js.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-L", libdir, "-ljscan", f"-Wl,-rpath,{libdir}",
           "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("c abi ok")
