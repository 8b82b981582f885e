"""Host-side checks of bench.py (no GPU): the one-GPU refusal, the algorithmic byte and flop
counts it prices the rooflines with, and the traffic summaries it reads.

The byte counts are restated here from the workload definitions (each input read once, each
output written once), the flop count from the contract's operation list (a decay multiply,
two 16-leaf dots and a rank-1 fma per state element and token, plus the delta's two ops per
row)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from bitwise_consistent_linear_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_flops_per_token_head_matches_the_operation_list():
    dk = dv = 128
    # per row: d_k decay muls; two dots of 16 leading muls, d_k - 16 fmas (2 flop) and 15
    # adds; delta sub and mul; d_k update fmas
    dot = 16 + 2 * (dk - 16) + 15
    per_row = dk + 2 * dot + 2 + 2 * dk
    assert per_row == 7 * dk
    assert bench.flops_per_token_head(dk, dv) == per_row * dv


def test_trainer_scan_bytes_count_each_input_and_output_once():
    w = W.trainer_fwd()
    T, Hk, Hv, d = w.total_tokens, w.num_qk_heads, w.num_v_heads, w.d_k
    q_k = 2 * T * Hk * d * 2           # bf16 q and k
    v = T * Hv * d * 2                 # bf16 v
    a_b = 2 * T * Hv * 4               # fp32 a and b
    cu = (w.num_seqs + 1) * 4          # cu_seqlens
    o = T * Hv * d * 4                 # fp32 o
    states = w.total_chunks * Hv * d * d * 4
    assert bench.scan_bytes(w, chunk_states=w.total_chunks) == q_k + v + a_b + cu + o + states
    assert w.total_chunks == 4 * 4096 // 64


def test_decode_step_bytes():
    N, Hk, Hv, d, C = 256, 16, 32, 128, 64
    state = N * Hv * d * d * 4
    expect = 2 * state + 2 * N * Hk * d * 2 + N * Hv * d * 2 + 2 * N * Hv * 4 + N * 4 \
        + N * Hv * d * 4 + state / C
    assert bench.decode_step_bytes(N, Hk, Hv, d, d, 2, C) == expect


@pytest.mark.parametrize("name", sorted(bench.KERNEL_SOURCES))
def test_traffic_summaries_are_well_formed(name):
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    with open(path) as f:
        t = json.load(f)
    assert t["hbm_bytes_per_launch"] == t["hbm_fetch_bytes_per_launch"] + \
        t["hbm_write_bytes_per_launch"] or \
        abs(t["hbm_bytes_per_launch"] - t["hbm_fetch_bytes_per_launch"]
            - t["hbm_write_bytes_per_launch"]) <= 1
    assert t["calibration_copy_bytes"] == bench.COPY_PROBE_BYTES
    # the scales come from the copy's own counter readings
    assert abs(t["fetch_scale"] - bench.COPY_PROBE_BYTES / (t["calibration_fetch_kib"] * 1024)) < 1e-3
    assert abs(t["write_scale"] - bench.COPY_PROBE_BYTES / (t["calibration_write_kib"] * 1024)) < 1e-3
    # measured traffic is at least the algorithmic bytes, up to counter noise
    assert t["hbm_bytes_per_launch"] >= 0.97 * t["algorithmic_bytes_per_launch"]
    # bench.py uses a summary only while the kernel sources hash to the recorded value
    used = bench.traffic_for(name)
    if t["kernel_source_sha256"] == bench.kernel_source_digest(name):
        assert used == t["hbm_bytes_per_launch"]
    else:
        assert used is None


def test_alu_peak_is_the_published_fp32_vector_peak():
    # 256 CUs x 4 SIMDs x 2.4 GHz x 64 flop per SIMD-cycle (two lanes' fused multiply-add
    # rate, which plain binary32 code reaches when two waves share a SIMD's issue slots)
    assert bench.FP32_VECTOR_PEAK_TFLOPS == 157.3
    assert abs(256 * 4 * 2.4e9 * 64 / 1e12 - bench.FP32_VECTOR_PEAK_TFLOPS) < 0.05
    r = bench.roofline_alu(157.3e12 * 1e-3, 2.0)  # half the peak
    assert r["peak"] == 157.3 and abs(r["frac"] - 0.5) < 1e-4 and r["bound"] == "alu"


def test_scan_kernel_names_are_matched_by_case():
    # the names rocprofv3 prints for the scan kernels (template: d_k, lanes per row, stage
    # tokens, bf16, case, threads per workgroup, rows per group of lanes)
    trainer = "void gdn::(anonymous namespace)::cpr_scan_kernel<128, 16, 64, true, 0, 512, 1>(gdn::ScanArgs)"
    prefill = "void gdn::(anonymous namespace)::cpr_scan_kernel<128, 4, 16, true, 1, 256, 2>(gdn::ScanArgs)"
    assert bench.is_scan_kernel(trainer, 0) and not bench.is_scan_kernel(trainer, 1)
    assert bench.is_scan_kernel(prefill, 1) and not bench.is_scan_kernel(prefill, 0)
    assert not bench.is_scan_kernel(
        "void gdn::(anonymous namespace)::cpr_decode_kernel<128, 16, true>(gdn::DecodeArgs)", 0)
