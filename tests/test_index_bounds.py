"""Bounds-checked host build of the launches' index arithmetic (no GPU).

sparse_attention_chunk_amd/csrc/fm_index.h holds the index functions the
kernels call: the score grid's wave shares and pipeline runs, the ragged
plan, the threshold mask words of a run, the top-K scan's tile size and
tile-word rows.  tests/index_check/check_index.cpp compiles that header
for the host with bounds-checked containers and the address and
undefined-behaviour sanitizers, and walks every run, mask word and tile word
over full, ragged, empty and long rows (see its header for the checks).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_chunk_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "index_check", "check_index.cpp")


def test_launch_index_arithmetic_stays_in_bounds(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / "check_index")
    build = subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                            "-fno-sanitize-recover=all", "-D_GLIBCXX_ASSERTIONS", "-I", CSRC, SRC, "-o", exe],
                           capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert run.stdout.startswith("checked "), run.stdout
