"""Host-side launch plans, checked on the CPU with the code the launchers run:
the plan header is plain C++ (no HIP), compiled here with the system C++
compiler into a small checker."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_precision_requant_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")


def _run_checker(name, tmp_path):
    exe = str(tmp_path / name)
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", f"-I{CSRC}", os.path.join(HOST, name + ".cpp"),
                    "-o", exe], check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    return r.returncode, r.stdout.strip()


def test_w4a16_register_decode_plan_fits_lds(tmp_path):
    """Every m <= 16 with K % 256 != 0 (the register-decode kernel) gets an
    instantiated pass length whose activation staging fits the 160 KB LDS --
    including shapes where the largest fitting pass is odd (e.g. m=12, n=4096,
    k=6016), which must round down, not up past the LDS size."""
    rc, out = _run_checker("w4a16_plan_check", tmp_path)
    assert rc == 0, out
    assert out.startswith("ok ")
    assert int(out.split()[1]) > 100000


def test_gemm_split_plan(tmp_path):
    """The K-split plan covers K with non-empty slices of whole stages, keeps the
    grid within two workgroups per CU and the workspace within its 8 MiB bound
    (which sizes the allocation-free entry point's static scratch)."""
    rc, out = _run_checker("split_plan_check", tmp_path)
    assert rc == 0, out
    assert out.startswith("ok ")
    cases, split = map(int, out.split()[1:])
    assert split > 1000 and cases > split


def test_gemm_big_tile_choice(tmp_path):
    """The 256 x 128 tile runs only on grids of at least two 128 x 128 tiles per
    CU, only where its tiling pads M no more than 128-row tiles, and only for
    K whose 256 rows fit 32-bit offsets; the prefill workloads take it."""
    rc, out = _run_checker("gemm_plan_check", tmp_path)
    assert rc == 0, out
    assert out.startswith("ok ")
    cases, tall = map(int, out.split()[1:])
    assert tall > 1000 and cases > tall
