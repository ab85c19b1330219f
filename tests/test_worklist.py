"""Host check of the verify kernel's work list (worklist.h): compiled with the
host compiler and run on the CPU, no GPU needed."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_worklist_covers_every_item_once_in_dependency_order(tmp_path):
    src = os.path.join(HERE, "native", "worklist_check.cpp")
    exe = str(tmp_path / "worklist_check")
    cc = subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror", src, "-o", exe],
                        capture_output=True, text=True)
    if cc.returncode != 0:
        pytest.fail("compile failed:\n" + cc.stderr)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")
