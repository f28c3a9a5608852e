"""The boundary from plain C: tests/c/abi_check.c, compiled with gcc against include/lynx.h and
linked against liblynx.so, runs the host-side size queries and validation paths (CPU only)."""
import os
import shutil
import subprocess

import pytest

from decode_attention_lynx_amd import lynx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_uses_the_abi(tmp_path):
    lib_dir = os.path.dirname(lynx.LIB_PATH)
    assert os.path.exists(lynx.LIB_PATH), "build the library first"
    exe = tmp_path / "abi_check"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_check.c"), "-L", lib_dir, "-llynx",
                    f"-Wl,-rpath,{lib_dir}", "-o", str(exe)], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"
