"""The decode tile pipeline's visiting order, checked on the host (CPU only).

tile_schedule (gqa_paged_kv_attention_amd/csrc/tile_schedule.h) is the integer
logic that every decode wave runs to decide which tile's page ids to fetch,
which register set to load and which tile to compute.  tests/
tile_schedule_check.cpp drives that same function with recording callbacks
over every range and stride a 4-wave work-group produces (both the paired and
the alternating double-buffered schedules, and the single-buffered one) and
checks that each tile is computed exactly once, from the registers loaded from
its own pages, with no page lookup outside the range.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_tile_schedule_visits_every_tile_once(tmp_path):
    inc = tmp_path / "include" / "hip"
    inc.mkdir(parents=True)
    (inc / "hip_runtime.h").write_text("#pragma once\n")       # the schedule needs nothing from HIP on the host
    exe = tmp_path / "tile_schedule_check"
    cmd = ["g++", "-std=c++17", "-O1", "-D__host__=", "-D__device__=", "-D__forceinline__=inline",
           "-I", str(tmp_path / "include"), "-I", os.path.join(ROOT, "gqa_paged_kv_attention_amd", "csrc"),
           os.path.join(ROOT, "tests", "tile_schedule_check.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
