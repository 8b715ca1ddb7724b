"""The C ABI from C: tests/c_client/abi_host.c includes only include/pkv.h, is compiled as strict
C99 and linked to the built library, then run. It covers the allocator, slot mapping, slot
validation, a short scheduler run, host-side refusals of device entry points (no pointer is
dereferenced, nothing reaches a GPU) and the per-thread failure message.
"""
import os
import shutil
import subprocess

import pytest

from prefill_slot_mapping_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_client", "abi_host.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c99_client_against_header(tmp_path):
    libdir, libname = os.path.split(os.path.abspath(L.LIB_PATH))
    exe = str(tmp_path / "abi_host")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), SRC, "-o", exe,
           "-L", libdir, f"-l:{libname}", f"-Wl,-rpath,{libdir}", "-pthread"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("ok ")
