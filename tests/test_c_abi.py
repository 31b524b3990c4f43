"""include/gdn.h compiles as C99 and libgdn.so links and answers from C (validation
paths only: no GPU is touched)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_program_links_and_validates(tmp_path):
    from gated_delta_rule_69_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from gated_delta_rule_69_amd import build
        build.build()
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(_lib.LIB_PATH)
    cmd = [cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi", "abi_check.c"), "-L", libdir,
           f"-Wl,-rpath,{libdir}", "-l:libgdn.so", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_check ok" in r.stdout
