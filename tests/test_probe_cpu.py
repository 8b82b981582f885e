"""libgdn_probe.so on the host: its exports and argument checks. No GPU is touched: every
call here is refused before anything is launched (fake pointers are never read)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "bitwise_consistent_linear_amd", "libgdn_probe.so")
FAKE = 0x1000  # a non-null address that no refused call dereferences


@pytest.fixture(scope="module")
def P():
    if not os.path.exists(PROBE):
        pytest.fail(f"{PROBE} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(PROBE)
    L.gdn_probe_valu.restype = ctypes.c_int
    L.gdn_probe_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p]
    L.gdn_probe_mfma.restype = ctypes.c_int
    L.gdn_probe_mfma.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 4 + [ctypes.c_int,
                                                                         ctypes.c_void_p]
    L.gdn_probe_valu_insts_per_iter.restype = ctypes.c_int
    return L


def test_exports():
    out = subprocess.run(["nm", "-D", "--defined-only", PROBE], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(gdn_\w+)$", out, flags=re.M))
    assert exported == {"gdn_probe_valu", "gdn_probe_valu_insts_per_iter", "gdn_probe_mfma"}


def test_every_form_issues_the_same_instruction_count(P):
    # bench.py divides every form's time by this one count
    assert P.gdn_probe_valu_insts_per_iter() == 128


@pytest.mark.parametrize("form,wps,iters,out,clk", [
    (-1, 1, 1, FAKE, FAKE), (5, 1, 1, FAKE, FAKE),      # forms 0..4 only
    (0, 0, 1, FAKE, FAKE), (3, 17, 1, FAKE, FAKE),      # 1..16 waves per SIMD
    (4, 1, 0, FAKE, FAKE),                              # at least one iteration
    (1, 1, 1, None, FAKE), (2, 1, 1, FAKE, None),       # both buffers
])
def test_valu_probe_refuses(P, form, wps, iters, out, clk):
    assert P.gdn_probe_valu(form, wps, iters, out, clk, None) == -1


@pytest.mark.parametrize("form,k,ptrs", [
    (2, 4, (FAKE,) * 4),                 # forms 0 and 1 only
    (0, 6, (FAKE,) * 4),                 # 16x16x4 takes K in steps of 4
    (1, 3, (FAKE,) * 4),                 # 32x32x2 takes K in steps of 2
    (0, 0, (FAKE,) * 4), (1, 258, (FAKE,) * 4),         # 1 <= K <= 256
    (0, 4, (None, FAKE, FAKE, FAKE)), (1, 2, (FAKE, FAKE, FAKE, None)),
])
def test_mfma_probe_refuses(P, form, k, ptrs):
    assert P.gdn_probe_mfma(form, *ptrs, k, None) == -1
