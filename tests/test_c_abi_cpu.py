"""The C ABI from plain C: include/mcs.h compiles as strict C99 and as C++17,
and a C program linked against the in-tree libmcs.so makes the host-only calls
and argument checks of tests/c_abi/abi_host_calls.c (no GPU needed)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
SRC = os.path.join(ROOT, "tests", "c_abi", "abi_host_calls.c")
PKG = os.path.join(ROOT, "sparse_attention_diffusion_mcs_amd")
LIB = os.path.join(PKG, "libmcs.so")


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not found")


def test_header_compiles_as_c99_and_cpp17(tmp_path):
    _need("gcc")
    _need("g++")
    src = tmp_path / "h.c"
    src.write_text('#include "mcs.h"\nint main(void) { return MCS_SUCCESS; }\n')
    for cc, std in (("gcc", "-std=c99"), ("g++", "-std=c++17")):
        r = subprocess.run([cc, std, "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INCLUDE, "-x",
                            "c" if cc == "gcc" else "c++", str(src), "-o", str(tmp_path / f"h_{cc}")],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr


def test_c_program_calls_the_library(tmp_path):
    _need("gcc")
    if not os.path.exists(LIB):
        pytest.skip("libmcs.so not built")
    exe = tmp_path / "abi_host_calls"
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INCLUDE, SRC, "-o",
                        str(exe), "-L", PKG, "-lmcs", f"-Wl,-rpath,{PKG}"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks held" in r.stdout
