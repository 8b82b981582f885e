"""Index arithmetic of cpr_io.hpp compiled for the host with hipcc: the scan's chunk-state
index (full_chunks, clamp_chunk_index) on adversarial cu_seqlens stays in [0, total_chunks]
even where a 32-bit sum of the chunk counts would wrap; the workgroup map (block_work) is a
bijection onto (pair, row block) and keeps each sequence's q/k-head group on one XCD."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def index_cases(tmp_path_factory):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("idx") / "index_arith")
    src = os.path.join(ROOT, "tests", "index_arith.cpp")
    csrc = os.path.join(ROOT, "bitwise_consistent_linear_amd", "csrc")
    subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17",
                    "-I", csrc, "-o", exe, src], check=True, capture_output=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    cases = {}
    for line in out.splitlines():
        _, name, *kv = line.split()
        cases[name] = {k: int(v) for k, v in (x.split("=") for x in kv)}
    assert cases, out
    return cases


def test_overlapping_ranges_clamp(index_cases):
    c = index_cases["overlapping_full_ranges"]
    # 2^15 full ranges of floor((2^31 - 1) / 16) chunks sum past 2^31: the index clamps
    assert c["first"] == 0
    assert 0 <= c["last"] <= c["total"] and c["max"] == c["total"]


def test_negative_and_decreasing_entries(index_cases):
    c = index_cases["negative_and_decreasing"]
    assert c["first"] == 0 and 0 <= c["max"] <= c["total"]


def test_plain_prefix_sums(index_cases):
    # lengths 64, 0, 136, 800 at C = 64: first states at 0, 1, 1, 3
    c = index_cases["plain"]
    assert (c["first"], c["last"], c["max"]) == (0, 3, 3)


def test_workgroup_map_is_a_bijection_that_keeps_groups_together(index_cases):
    maps = {k: v for k, v in index_cases.items() if k.startswith("map_")}
    assert len(maps) == 10
    for name, c in maps.items():
        assert c["bijective"] == 1, name
        assert c["together"] == 1, name
