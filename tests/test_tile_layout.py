"""The LDS tile layouts of the 16-bit kernels, checked on the host.

tests/tile_layout_check.cpp includes the kernels' own header and checks, for every lane, that the
DMA placement and the row / transposing read offsets agree byte for byte and that the lanes of
one LDS transfer hit distinct banks.  A second build against a copy of the header with a planted
mistake (the run stride of the D = 128 layout set to 1024, which puts four rows of a
transposing read on the same banks) must fail it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "variable_length_flashattention_fa_amd", "csrc")
CHECK_SRC = os.path.join(ROOT, "tests", "tile_layout_check.cpp")


def _hipcc():
    return os.environ.get("HIPCC") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc")
                                       else shutil.which("hipcc"))


def _build_and_run(csrc_dir, out_dir):
    hipcc = _hipcc()
    if not hipcc:
        pytest.skip("hipcc not available")
    exe = os.path.join(out_dir, "tile_layout_check")
    cmd = [hipcc, "-std=c++17", "-O1", "-x", "hip", "--cuda-host-only", f"-I{os.path.join(ROOT, 'include')}",
           f"-I{csrc_dir}", CHECK_SRC, "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    return subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=60)


def test_tile_layouts_match_reads_and_avoid_bank_conflicts(tmp_path):
    r = _build_and_run(CSRC, str(tmp_path))
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout


def test_checker_catches_a_wrong_run_stride(tmp_path):
    bad = tmp_path / "csrc"
    shutil.copytree(CSRC, bad, ignore=shutil.ignore_patterns("__pycache__", "*.o"))
    hdr = bad / "fa_device.h"
    text = hdr.read_text()
    assert "static constexpr int kRunBytes = 1040;" in text
    hdr.write_text(text.replace("static constexpr int kRunBytes = 1040;", "static constexpr int kRunBytes = 1024;"))
    r = _build_and_run(str(bad), str(tmp_path))
    assert r.returncode == 1 and "failures" in r.stdout, r.stdout
