"""The decode tile pipeline's visiting order and the decode grid's work-group
pairing, checked on the host (CPU only).

tile_schedule (gqa_paged_kv_attention_amd/csrc/tile_schedule.h) is the integer
logic that every decode wave runs to decide which tile's page ids to fetch,
which register set to load and which tile to compute.  tests/
tile_schedule_check.cpp drives that same function with recording callbacks
over every range and stride a 4-wave work-group produces (both the paired and
the alternating double-buffered schedules, and the single-buffered one) and
checks that each tile is computed exactly once, from the registers loaded from
its own pages, with no page lookup outside the range.

paired_unit (csrc/work_map.h) maps the decode grid's work-groups to units
when each kv head's query heads run as two units: tests/work_map_check.cpp
checks that it is one to one for every even grid size up to 4096 and that the
two halves of a unit share an XCD wherever the map promises it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_host_check(tmp_path, name):
    inc = tmp_path / "include" / "hip"
    inc.mkdir(parents=True, exist_ok=True)
    (inc / "hip_runtime.h").write_text("#pragma once\n")       # the logic needs nothing from HIP on the host
    exe = tmp_path / name
    cmd = ["g++", "-std=c++17", "-O1", "-D__host__=", "-D__device__=", "-D__forceinline__=inline",
           "-I", str(tmp_path / "include"), "-I", os.path.join(ROOT, "gqa_paged_kv_attention_amd", "csrc"),
           os.path.join(ROOT, "tests", name + ".cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_tile_schedule_visits_every_tile_once(tmp_path):
    _run_host_check(tmp_path, "tile_schedule_check")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_paired_units_are_one_to_one_and_share_an_xcd(tmp_path):
    _run_host_check(tmp_path, "work_map_check")
