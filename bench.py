"""Benchmark of the CPR Gated DeltaNet hot path on one MI355X.

Prints ONE JSON line on stdout (progress goes to stderr). The headline step is one
trainer_fwd call (gdn_cpr_trainer_fwd: every token's o plus the state at every 64-token
boundary) over the trainer workload: 4 sequences x 4096 tokens, 16 heads, d_k = d_v = 128,
C = 64, bf16 q/k/v, fp32 a/b/state/o. `value` is tokens/s of that step with inputs already
in HBM. The same line also reports, under "cases", engine_prefill tokens/s (64 varlen
sequences, 262144 tokens, 16 q/k / 32 v heads), the engine_decode step time (256
sequences after a 1000-token prefill, 512 steps), the backward (gdn_cpr_trainer_bwd) on
the trainer workload, the long-context runs, the linear region (a 16384 x 4096 x 4096
batch-invariant matrix product on the matrix cores) and the two-level reading of CPR
(chunk transitions, a boundary sweep on the matrix cores, outputs), each with its
fraction of the relevant peak, plus the CPU oracle timed on the host as a baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--cases all|main|bwd|linear|cpr2|traffic]
                       [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0             # MI355X HBM3E, spec sheet
# fp32 vector peak: 256 CU x 4 SIMD x 2.4 GHz x 64 flop per SIMD-cycle. The kernels emit no
# packed fp32; gfx950 still reaches this rate with plain instructions when two waves on a
# SIMD issue one vector instruction each in the same four-cycle slot (measured by the probe
# beside every run: valu_probe in the JSON line).
FP32_VECTOR_PEAK_TFLOPS = 157.3
FP32_MFMA_PEAK_TFLOPS = 157.3     # dense binary32 matrix instructions (the linear region)
METRIC = "GDN-CPR tokens/s (trainer_fwd, prefill), decode-step us, % of HBM peak"
KERNEL_SOURCES = {  # sources whose hash a traffic summary must match to be used
    "cpr_scan_trainer_fwd": ["cpr_kernels.hip", "cpr_row.hpp", "cpr_io.hpp"],
    "cpr_scan_engine_prefill": ["cpr_kernels.hip", "cpr_row.hpp", "cpr_io.hpp"],
    "cpr_scan_long_context_trainer": ["cpr_kernels.hip", "cpr_row.hpp", "cpr_io.hpp"],
    "cpr_scan_long_context_prefill": ["cpr_kernels.hip", "cpr_row.hpp", "cpr_io.hpp"],
    "cpr_decode_engine_decode": ["cpr_kernels.hip", "cpr_row.hpp", "cpr_io.hpp"],
    "cpr_bwd_trainer": ["cpr_backward.hip", "cpr_row.hpp", "cpr_io.hpp"],
    "cpr2_two_level_trainer": ["cpr2.hip", "cpr_row.hpp", "cpr_io.hpp"],
    "linear_leaf_16384x4096x4096": ["linear.hip"],
}
PMC_COMMAND = ("rocprofv3 --pmc {counter} --output-format csv -d <dir> -o {name} -- python3 "
               "bench.py --cases traffic --no-cpu-baseline --steps 3 --warmup 1 --copy-probe")
COPY_PROBE_BYTES = 256 << 20  # read once and written once by the calibration copy


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_digest(name="cpr_scan_trainer_fwd"):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name]:
        with open(os.path.join(ROOT, "bitwise_consistent_linear_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def flops_per_token_head(dk, dv):
    # per row and token: decay d_k mul; two contract dots of 16 mul + (d_k-16) fma + 15 add
    # = 2 d_k - 1 flop each; delta 2; rank-1 update d_k fma = 2 d_k  ->  7 d_k flop
    return 7 * dk * dv


def bwd_flops_per_token_head(dk, dv):
    # per row and token, in the backward contract's order: one recompute of the forward
    # state (decay d_k, dot 2 d_k - 1, delta 2, update 2 d_k: 5 d_k + 1); the backward's own
    # work: sh += g q (2 d_k), pq = g s (d_k), dh = dot (2 d_k - 1), dv and pb (2),
    # xh (2 d_k), pk (3 d_k), pa = dot (2 d_k - 1), sh = a xh (d_k): 13 d_k; the row sums of
    # dq and dk (2 d_k adds per row) -> 20 d_k flop, rounded down
    return 20 * dk * dv


def bwd_bytes(w):
    """Algorithmic HBM bytes of one backward call: inputs (q, k, v, a, b, d_o, d_final_state,
    the chunk states) read once, outputs (dq, dk, dv, da, db, dS0) written once."""
    el = 2 if w.bf16 else 4
    T, Hk, Hv, dk, dv, N = w.total_tokens, w.num_qk_heads, w.num_v_heads, w.d_k, w.d_v, w.num_seqs
    state = Hv * dv * dk * 4
    reads = (T * Hk * dk * el * 2 + T * Hv * dv * el + T * Hv * 4 * 2 + T * Hv * dv * 4
             + (w.total_chunks + N) * state + (N + 1) * 4)
    writes = T * Hk * dk * 4 * 2 + T * Hv * dv * 4 + T * Hv * 4 * 2 + N * state
    return reads + writes


def scan_bytes(w, with_o=True, chunk_states=0, final_states=0, initial_states=0):
    """Algorithmic HBM bytes of one scan call: each input read once, each output written once."""
    el = 2 if w.bf16 else 4
    T, Hk, Hv, dk, dv = w.total_tokens, w.num_qk_heads, w.num_v_heads, w.d_k, w.d_v
    b = T * Hk * dk * el * 2 + T * Hv * dv * el + T * Hv * 4 * 2 + (w.num_seqs + 1) * 4
    if with_o:
        b += T * Hv * dv * 4
    b += (chunk_states + final_states + initial_states) * Hv * dv * dk * 4
    return b


def cpr2_bytes(w):
    """Algorithmic HBM bytes of one two-level trainer call: the inputs once, o once, the
    chunk states written once and read once (the outputs restart from them), and the
    transitions A_c, B_c written once and read once."""
    trans = w.total_chunks * w.num_v_heads * (w.d_k + w.d_v) * w.d_k * 4
    states = w.total_chunks * w.num_v_heads * w.d_v * w.d_k * 4
    return scan_bytes(w, chunk_states=w.total_chunks) + states + 2 * trans


def decode_step_bytes(N, Hk, Hv, dk, dv, el, C):
    state = N * Hv * dv * dk * 4
    return (2 * state + N * Hk * dk * el * 2 + N * Hv * dv * el + N * Hv * 4 * 2 + N * 4
            + N * Hv * dv * 4 + state / C)


def up(x):
    import numpy as np
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(x).cuda()


def timed(fn, steps, warmup):
    """Run fn warmup times, then time `steps` calls: wall clock of the whole region and HIP
    events around each call on the current stream. Returns (wall_s, per_call_ms list)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for s, e in evs:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [s.elapsed_time(e) for s, e in evs]


def roofline_alu(flops, ms):
    achieved = flops / (ms * 1e-3) / 1e12
    return {"bound": "alu", "achieved": round(achieved, 3), "peak": FP32_VECTOR_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / FP32_VECTOR_PEAK_TFLOPS, 4)}


def same_bits(x, y):
    """Bitwise equality of two float32 device tensors (compared as int32 on the device)."""
    import torch
    return bool(torch.equal(x.contiguous().view(torch.int32), y.contiguous().view(torch.int32)))


def verdict(checks):
    """The parity verdict of one case: every check is a bitwise comparison on the device."""
    return {"bitwise_exact": all(checks.values()), "checks": checks}


def valu_probe():
    """Vector-issue ceiling and shader clock of this GPU, from libgdn_probe.so: SIMD-cycles
    per wave instruction for plain multiplies, fused multiply-adds, DPP adds and a single
    dependent chain of fused multiply-adds per lane with one, two and four waves per SIMD,
    the fused multiply-add rate at two waves per SIMD, the latency
    of a dependent fused multiply-add and of a dependent DPP add level (shader cycles per step
    of one chain per lane, one wave per SIMD), and the shader clock (s_memtime against the
    100 MHz s_memrealtime)."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "bitwise_consistent_linear_amd", "libgdn_probe.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.gdn_probe_valu.restype = ctypes.c_int
    L.gdn_probe_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p]
    per_iter = L.gdn_probe_valu_insts_per_iter()
    iters = 4000
    out = {"unit": "SIMD-cycles per wave instruction at the measured clock"}
    clocks = []
    fma2 = None
    for form, name in ((0, "v_mul_f32"), (1, "v_fmac_f32"), (2, "v_add_f32_dpp"),
                       (3, "v_fmac_f32_one_dependent_chain")):
        row = {}
        for wps in (1, 2, 4):
            grid = 256 * wps
            buf = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
            clk = torch.empty(grid * 2, dtype=torch.int64, device="cuda")
            stream = torch.cuda.current_stream().cuda_stream
            if L.gdn_probe_valu(form, wps, iters // 10, buf.data_ptr(), clk.data_ptr(), stream):
                return None
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if L.gdn_probe_valu(form, wps, iters, buf.data_ptr(), clk.data_ptr(), stream):
                return None
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            c = clk.view(grid, 2).double().sum(0)
            ghz = float(c[0] / (c[1] / 100e6) / 1e9)
            clocks.append(ghz)
            insts_per_simd = wps * iters * per_iter
            row[str(wps)] = round(ms * 1e-3 * ghz * 1e9 / insts_per_simd, 3)
            if form == 1 and wps == 2:
                fma2 = 2 * 64 * 1024 * insts_per_simd / (ms * 1e-3) / 1e12
        out[name] = row
    out["v_fmac_f32_TFLOPs_at_2_waves_per_simd"] = round(fma2, 1)
    # latency: one dependent chain per lane, one wave per SIMD, shader cycles per step
    for form, name in ((3, "dependent_v_fmac_f32"), (4, "dependent_dpp_add_level")):
        grid = 256
        buf = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
        clk = torch.empty(grid * 2, dtype=torch.int64, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        if L.gdn_probe_valu(form, 1, iters, buf.data_ptr(), clk.data_ptr(), stream):
            return None
        torch.cuda.synchronize()
        c = clk.view(grid, 2).double().sum(0)
        out[name + "_cycles_per_step"] = round(float(c[0]) / grid / (iters * per_iter), 2)
    out["shader_clock_GHz"] = round(sum(clocks) / len(clocks), 3)
    return out


def hbm(bytes_, ms):
    gbs = bytes_ / (ms * 1e-3) / 1e9
    return {"algorithmic_bytes": int(bytes_), "achieved_GBs": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def is_scan_kernel(name, mode):
    """Whether a kernel name from a profile is a one-level scan of the case `mode` (0 trainer,
    1 prefill): template arguments (d_k, lanes, stage tokens, bf16, case, threads, rows per
    group of lanes)."""
    return re.search(rf"cpr_scan_kernel<\d+, \d+, \d+, (true|false), {mode}, \d+, \d+>"
                     r"\(gdn::ScanArgs\)$", name) is not None


def traffic_for(name, launches_bytes_fn=None):
    """Measured HBM bytes per launch from a committed rocprofv3 counter summary, if it was
    taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_digest(name):
        return None
    return int(t["hbm_bytes_per_launch"])


def write_traffic(fetch_csv, write_csv):
    """From two rocprofv3 --pmc runs of `bench.py --cases traffic --copy-probe` (FETCH_SIZE,
    then WRITE_SIZE; KiB per dispatch), write profiles/<name>_traffic.json for every one-level
    scan case, the decode step, the backward, the two-level trainer and the linear region:
    HBM bytes per launch (per call for the multi-kernel ones), each counter scaled by what
    it reads for the 256 MiB calibration copy (read once, written once)."""
    import csv
    import statistics

    def rows(path, counter):
        return [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]

    def copy_kib(rs):
        # the calibration copies are the first device-to-device copies of the run: --copy-probe
        # makes them right after the library loads, before any upload
        cp = sorted((int(r["Dispatch_Id"]), float(r["Counter_Value"])) for r in rs
                    if "copyBuffer" in r["Kernel_Name"])
        c = [v for _, v in cp[:3]]
        if len(c) < 3 or min(c) < 1024:
            raise SystemExit("no calibration copy in the counter files")
        return statistics.median(c)

    def per_kernel(rs, match):
        by = {}
        for r in rs:
            if match(r["Kernel_Name"], int(r["Grid_Size"])):
                by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: statistics.median(v) for k, v in by.items()}

    def scan(mode, grid):  # one scan launch of the case at that many threads
        return lambda name, g: is_scan_kernel(name, mode) and g == grid

    fr, wr = rows(fetch_csv, "FETCH_SIZE"), rows(write_csv, "WRITE_SIZE")
    cf, cw = copy_kib(fr), copy_kib(wr)
    fetch_scale = COPY_PROBE_BYTES / (cf * 1024)
    write_scale = COPY_PROBE_BYTES / (cw * 1024)
    from bitwise_consistent_linear_amd import workloads as W
    w = W.trainer_fwd()
    wp, wl, wd = W.engine_prefill(), W.long_context(), W.engine_decode()
    threads = 256

    def grid(wk, lanes, per_group=1):  # threads of a one-level launch at `lanes` lanes per row
        rows = per_group * (threads // lanes)
        return wk.num_seqs * wk.num_v_heads * -(-wk.d_v // rows) * threads

    dec_state = wd.num_seqs * wd.num_v_heads * wd.d_v * wd.d_k * 4
    targets = [
        ("cpr_scan_trainer_fwd", scan(0, grid(w, 16)),
         "trainer_fwd: 4 x 4096 tokens, 16 heads, d=128, C=64, bf16 q/k/v",
         scan_bytes(w, chunk_states=w.total_chunks)),
        ("cpr_scan_engine_prefill", scan(1, grid(wp, 4, 2)),
         "engine_prefill: 64 varlen sequences, 262144 tokens, 16 q/k / 32 v heads, d=128, "
         "bf16 q/k/v; o and the final states", scan_bytes(wp, final_states=wp.num_seqs)),
        ("cpr_scan_long_context_trainer", scan(0, grid(wl, 16)),
         "long_context trainer_fwd: 1 x 131072 tokens, 16 q/k / 32 v heads, d=128, C=64",
         scan_bytes(wl, chunk_states=wl.total_chunks)),
        ("cpr_scan_long_context_prefill", scan(1, grid(wl, 16)),
         "long_context prefill: 1 x 131072 tokens, 16 q/k / 32 v heads, d=128",
         scan_bytes(wl, final_states=1)),
        ("cpr_decode_engine_decode",
         lambda name, g: "cpr_decode_kernel<" in name and g == grid(wd, 16),
         "engine_decode: one decode step of 256 sequences, 16 q/k / 32 v heads, d=128, C=64 "
         "(per step; a step that ends no chunk writes no resync checkpoint)",
         decode_step_bytes(wd.num_seqs, wd.num_qk_heads, wd.num_v_heads, wd.d_k, wd.d_v, 2,
                           wd.chunk) - dec_state / wd.chunk),
        ("cpr_bwd_trainer", lambda name, g: "cpr_bwd_" in name,
         "trainer_bwd on the trainer_fwd workload (every backward kernel of one call)",
         bwd_bytes(w)),
        ("cpr2_two_level_trainer", lambda name, g: "cpr2_" in name,
         "two-level trainer_fwd on the trainer_fwd workload (every kernel of one call)",
         cpr2_bytes(w)),
        ("linear_leaf_16384x4096x4096",
         lambda name, g: "linear_leaf_kernel<" in name and g == LINEAR_GRID_THREADS,
         "linear region: Y[16384, 4096] = X[16384, 4096] W[4096, 4096], bf16 X and W, "
         "binary32 Y", linear_bytes(16384, 4096, 4096)),
    ]
    for name, match, workload, alg in targets:
        kf, kw = per_kernel(fr, match), per_kernel(wr, match)
        if not kf or not kw:
            raise SystemExit(f"no dispatch for {name} in the counter files")
        kernels = {k: {"fetch_kib": kf[k], "write_kib": kw.get(k, 0.0),
                       "hbm_bytes": int(kf[k] * 1024 * fetch_scale
                                        + kw.get(k, 0.0) * 1024 * write_scale)}
                   for k in sorted(kf)}
        fetch_b = sum(v["fetch_kib"] for v in kernels.values()) * 1024 * fetch_scale
        write_b = sum(v["write_kib"] for v in kernels.values()) * 1024 * write_scale
        out = {
            "kernels": kernels,
            "workload": workload,
            "kernel_source_sha256": kernel_source_digest(name),
            "calibration_copy_bytes": COPY_PROBE_BYTES,
            "calibration_fetch_kib": cf, "calibration_write_kib": cw,
            "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
            "hbm_fetch_bytes_per_launch": int(fetch_b),
            "hbm_write_bytes_per_launch": int(write_b),
            "hbm_bytes_per_launch": int(fetch_b + write_b),
            "algorithmic_bytes_per_launch": int(alg),
            "commands": [PMC_COMMAND.format(counter="FETCH_SIZE", name="fetch"),
                         PMC_COMMAND.format(counter="WRITE_SIZE", name="write"),
                         "python3 bench.py --traffic-from <dir>/fetch_counter_collection.csv "
                         "<dir>/write_counter_collection.csv"],
        }
        path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
        with open(path, "w") as f:
            json.dump(out, f, indent=1)
            f.write("\n")
        print(name, out["hbm_bytes_per_launch"], "bytes per launch;",
              out["algorithmic_bytes_per_launch"], "algorithmic")


# ------------------------------------------------------------------------------ cases

def bench_trainer(steps, warmup):
    import torch
    from bitwise_consistent_linear_amd import api
    from bitwise_consistent_linear_amd import workloads as W
    w = W.trainer_fwd()
    log(f"trainer_fwd: N={w.num_seqs} T={w.lengths[0]} H={w.num_v_heads} d={w.d_k} C={w.chunk}")
    cu, q, k, v, a, b = (up(x) for x in (w.cu_seqlens, w.q, w.k, w.v, w.a, w.b))
    o = torch.empty((w.total_tokens, w.num_v_heads, w.d_v), dtype=torch.float32, device="cuda")
    cs = torch.empty((w.total_chunks, w.num_v_heads, w.d_v, w.d_k), dtype=torch.float32,
                     device="cuda")
    tc = w.total_chunks

    def step():
        api.trainer_fwd(cu, q, k, v, a, b, chunk=w.chunk, o=o, chunk_states=cs, total_chunks=tc)

    wall, per = timed(step, steps, warmup)
    kernel_ms = sum(per) / len(per)
    flops = flops_per_token_head(w.d_k, w.d_v) * w.total_tokens * w.num_v_heads
    nbytes = scan_bytes(w, chunk_states=tc)
    # parity, after the timed region: the prefill case on the same batch, and a repeat
    po, fs = api.prefill(cu, q, k, v, a, b, chunk=w.chunk)
    o2, cs2 = api.trainer_fwd(cu, q, k, v, a, b, chunk=w.chunk, total_chunks=tc)
    torch.cuda.synchronize()
    N, Tn = w.num_seqs, int(w.lengths[0])
    last = cs.view(N, Tn // w.chunk, w.num_v_heads, w.d_v, w.d_k)[:, -1]
    par = verdict({"prefill o == trainer o": same_bits(po, o),
                   "prefill final state == trainer last chunk state": same_bits(fs, last),
                   "repeat call: same o and chunk states": same_bits(o2, o) and same_bits(cs2, cs)})
    outputs = (o.cpu().numpy(), cs.cpu().numpy())
    del po, fs, o2, cs2, q, k, v, o, cs
    return w, wall, kernel_ms, flops, nbytes, par, outputs


def bench_prefill(steps, warmup):
    import numpy as np
    import torch
    from bitwise_consistent_linear_amd import api
    from bitwise_consistent_linear_amd import workloads as W
    w = W.engine_prefill()
    L = w.lengths
    log(f"engine_prefill: N={w.num_seqs} lengths {L.min()}..{L.max()} sum {L.sum()}")
    cu, q, k, v, a, b = (up(x) for x in (w.cu_seqlens, w.q, w.k, w.v, w.a, w.b))
    o = torch.empty((w.total_tokens, w.num_v_heads, w.d_v), dtype=torch.float32, device="cuda")
    fs = torch.empty((w.num_seqs, w.num_v_heads, w.d_v, w.d_k), dtype=torch.float32,
                     device="cuda")

    def step():
        api.prefill(cu, q, k, v, a, b, chunk=w.chunk, o=o, final_state=fs)

    wall, per = timed(step, steps, warmup)
    ms = sum(per) / len(per)
    flops = flops_per_token_head(w.d_k, w.d_v) * w.total_tokens * w.num_v_heads
    nbytes = scan_bytes(w, final_states=w.num_seqs)
    # parity, after the timed region: the trainer case's o on the same batch (no chunk states
    # requested), and the final state of every sequence whose length is a multiple of C
    # against its trainer's last chunk state
    to, tcs = api.trainer_fwd(cu, q, k, v, a, b, chunk=w.chunk, total_chunks=w.total_chunks)
    torch.cuda.synchronize()
    coff = np.concatenate([[0], np.cumsum(L // w.chunk)])
    whole = [n for n in range(w.num_seqs) if L[n] % w.chunk == 0 and L[n] > 0]
    fin = all(same_bits(fs[n], tcs[int(coff[n + 1]) - 1]) for n in whole)
    par = verdict({"trainer o == prefill o": same_bits(to, o),
                   f"final state == last chunk state ({len(whole)} sequences of whole chunks)":
                   fin})
    del q, k, v, o, to, tcs
    return {"workload": f"engine_prefill: 64 varlen sequences (lognormal, {L.min()}..{L.max()} "
                        f"tokens), {L.sum()} tokens, 16 q/k / 32 v heads, d=128, C=64, bf16 q/k/v",
            "tokens_per_s": round(w.total_tokens / (wall / steps), 1),
            "ms_per_call": round(wall / steps * 1e3, 4), "kernel_ms": round(ms, 4),
            "steps": steps,
            "roofline": dict(roofline_alu(flops, ms), traffic=traffic_for("cpr_scan_engine_prefill")),
            "hbm": hbm(nbytes, ms), "parity": par}


def bench_trainer_bwd(steps, warmup, fwd_kernel_ms, verify=True):
    """gdn_cpr_trainer_bwd on the trainer workload, given seeded dL/do and dL/dS_final."""
    import torch
    from bitwise_consistent_linear_amd import api
    from bitwise_consistent_linear_amd import workloads as W
    w = W.trainer_fwd()
    do, dsf = W.cotangents(w, 11)
    log("trainer_bwd: same workload, seeded dL/do and dL/dS_final")
    cu, q, k, v, a, b = (up(x) for x in (w.cu_seqlens, w.q, w.k, w.v, w.a, w.b))
    ddo, ddsf = up(do), up(dsf)
    tc = w.total_chunks
    _, cs = api.trainer_fwd(cu, q, k, v, a, b, chunk=w.chunk, total_chunks=tc)
    shape = api.GdnShape(w.num_seqs, w.num_qk_heads, w.num_v_heads, w.d_k, w.d_v, w.chunk,
                         api.GDN_DTYPE_BF16)
    need = api.trainer_bwd_workspace_bytes(shape, w.total_tokens, tc)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    grads = api.trainer_bwd(cu, q, k, v, a, b, cs, ddo, chunk=w.chunk, d_final_state=ddsf,
                            total_chunks=tc, workspace=ws)

    def step():
        api.trainer_bwd(cu, q, k, v, a, b, cs, ddo, chunk=w.chunk, d_final_state=ddsf,
                        total_chunks=tc, workspace=ws, out=grads)

    wall, per = timed(step, steps, warmup)
    ms = sum(per) / len(per)
    flops = bwd_flops_per_token_head(w.d_k, w.d_v) * w.total_tokens * w.num_v_heads
    if not verify:  # the counter runs: only the timed schedule's kernels
        del q, k, v, cs, ws, grads
        return {"kernel_ms": round(ms, 4)}
    # parity, after the timed region: a repeat, and the other schedule (a reverse state pass,
    # then every chunk in parallel), which must give the same bits
    again = api.trainer_bwd(cu, q, k, v, a, b, cs, ddo, chunk=w.chunk, d_final_state=ddsf,
                            total_chunks=tc, workspace=ws)
    sched = os.environ.get("GDN_CPR_BWD_SCHEDULE")
    os.environ["GDN_CPR_BWD_SCHEDULE"] = "chunks"
    try:
        other = api.trainer_bwd(cu, q, k, v, a, b, cs, ddo, chunk=w.chunk, d_final_state=ddsf,
                                total_chunks=tc, workspace=ws)
    finally:
        if sched is None:
            del os.environ["GDN_CPR_BWD_SCHEDULE"]
        else:
            os.environ["GDN_CPR_BWD_SCHEDULE"] = sched
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "da", "db", "dS0")
    par = verdict({"repeat call: same gradients": all(same_bits(again[g], grads[g]) for g in names),
                   "chunk schedule == sequence schedule": all(same_bits(other[g], grads[g])
                                                              for g in names)})
    del q, k, v, cs, ws, grads, again, other
    return {"workload": "trainer_bwd: the trainer_fwd workload (4 x 4096 tokens, 16 heads, "
                        "d=128, C=64, bf16 q/k/v) given dL/do and dL/dS_final; writes dq, dk, "
                        "dv, da, db, dS0",
            "tokens_per_s": round(w.total_tokens / (wall / steps), 1),
            "ms_per_call": round(wall / steps * 1e3, 4), "kernel_ms": round(ms, 4),
            "fwd_plus_bwd_kernel_ms": round(fwd_kernel_ms + ms, 4),
            "workspace_bytes": int(need), "steps": steps,
            "roofline": dict(roofline_alu(flops, ms), traffic=traffic_for("cpr_bwd_trainer")),
            "hbm": hbm(bwd_bytes(w), ms), "parity": par}


LINEAR_GRID_THREADS = (16384 // 128) * (4096 // 128) * 512  # the bench product's launch


def linear_bytes(M, N, K):
    """Algorithmic bytes of one linear-region call: bf16 X and W read once, binary32 Y
    written once."""
    return M * K * 2 + K * N * 2 + M * N * 4


def bench_linear(steps, warmup, M=16384, N=4096, K=4096):
    """gdn_linear_fwd: Y = X W with every output the contract dot, on the matrix cores."""
    import torch
    from bitwise_consistent_linear_amd import api
    from bitwise_consistent_linear_amd import workloads as W
    log(f"linear: {M} x {N} x {K}, bf16 inputs")
    x, w = W.make_linear(M, N, K, True, 31)
    dx, dw = up(x), up(w)
    y = api.linear_fwd(dx, dw)
    wall, per = timed(lambda: api.linear_fwd(dx, dw, y=y), steps, warmup)
    ms = sum(per) / len(per)
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    nbytes = linear_bytes(M, N, K)
    # parity, after the timed region: batch invariance - rows computed in a batch of 65
    # equal the same rows of the full product
    part = api.linear_fwd(dx[:65].contiguous(), dw)
    torch.cuda.synchronize()
    par = verdict({"rows of a 65-row batch == the same rows of the full batch":
                   same_bits(part, y[:65])})
    del dx, dw, y, part
    return {"workload": f"linear region: Y[{M}, {N}] = X[{M}, {K}] W[{K}, {N}], bf16 X and W "
                        "(widened exactly), binary32 Y, each output the 16-leaf contract dot",
            "ms_per_call": round(wall / steps * 1e3, 4), "kernel_ms": round(ms, 4),
            "steps": steps,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                         "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / FP32_MFMA_PEAK_TFLOPS, 4),
                         "traffic": traffic_for(f"linear_leaf_{M}x{N}x{K}")},
            "hbm": hbm(nbytes, ms), "parity": par}


def cpr2_flops(w):
    """Flops of one two-level call: each full chunk's transition runs d_k + d_v rows through
    the row update (5 d_k + 1 flop per row and token), its boundary step is a d_v x d_k x
    d_k multiply-add (on the matrix units), and the outputs repeat the recurrence from the
    boundary states (7 d_k per row and token, as in the one-level scan)."""
    dk, dv, C, Hv = w.d_k, w.d_v, w.chunk, w.num_v_heads
    trans = w.total_chunks * Hv * (dk + dv) * C * (5 * dk + 1)
    boundary = w.total_chunks * Hv * dv * dk * dk * 2
    outputs = flops_per_token_head(dk, dv) * w.total_tokens * Hv
    return trans, boundary, outputs


def bench_cpr2(steps, warmup, trainer_only=False):
    """The two-level reading of CPR (gdn_cpr2_*): trainer_fwd and prefill on the trainer
    workload, decode steps on the engine-decode workload from a chunk-aligned prefix
    (trainer_only: the trainer calls alone, for the counter runs)."""
    import torch
    from bitwise_consistent_linear_amd import api
    from bitwise_consistent_linear_amd import workloads as W
    w = W.trainer_fwd()
    log("cpr2: two-level trainer_fwd and prefill on the trainer workload")
    cu, q, k, v, a, b = (up(x) for x in (w.cu_seqlens, w.q, w.k, w.v, w.a, w.b))
    tc = w.total_chunks
    T, Hv, dv, dk = w.total_tokens, w.num_v_heads, w.d_v, w.d_k
    o = torch.empty((T, Hv, dv), dtype=torch.float32, device="cuda")
    cs = torch.empty((tc, Hv, dv, dk), dtype=torch.float32, device="cuda")
    fs = torch.empty((w.num_seqs, Hv, dv, dk), dtype=torch.float32, device="cuda")
    shape = api.GdnShape(w.num_seqs, w.num_qk_heads, Hv, dk, dv, w.chunk, api.GDN_DTYPE_BF16)
    need = api.cpr2_workspace_bytes(shape, T, tc, False)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    wall_t, per_t = timed(lambda: api.cpr2_trainer_fwd(cu, q, k, v, a, b, chunk=w.chunk, o=o,
                                                       chunk_states=cs, total_chunks=tc,
                                                       workspace=ws), steps, warmup)
    mt = sum(per_t) / len(per_t)
    trans, boundary, outputs = cpr2_flops(w)
    roof = roofline_alu(trans + boundary + outputs, mt)
    roof["scope"] = ("whole call (plan, transitions, boundary sweep, outputs); the boundary "
                     "sweep's flops run on the matrix units")
    roof["traffic"] = traffic_for("cpr2_two_level_trainer")
    if trainer_only:
        return {"trainer_fwd_kernel_ms": round(mt, 4), "steps": steps, "roofline": roof}
    po = torch.empty_like(o)
    wall_p, per_p = timed(lambda: api.cpr2_prefill(cu, q, k, v, a, b, chunk=w.chunk, o=po,
                                                   final_state=fs, total_chunks=tc,
                                                   workspace=ws), steps, warmup)
    mp = sum(per_p) / len(per_p)
    torch.cuda.synchronize()
    N, Tn = w.num_seqs, int(w.lengths[0])
    checks = {"two-level prefill o == two-level trainer o": same_bits(po, o),
              "two-level final state == last chunk state (whole chunks)":
              same_bits(fs, cs.view(N, Tn // w.chunk, Hv, dv, dk)[:, -1])}
    del q, k, v, o, po, cs, fs, ws
    torch.cuda.empty_cache()
    dec = bench_cpr2_decode()
    torch.cuda.empty_cache()
    big = {}
    for label, make, trainer in (("long_context_trainer", W.long_context, True),
                                 ("engine_prefill_prefill", W.engine_prefill, False)):
        wb = make()
        log(f"cpr2: {label}")
        d = [up(x) for x in (wb.cu_seqlens, wb.q, wb.k, wb.v, wb.a, wb.b)]
        shape_b = api.GdnShape(wb.num_seqs, wb.num_qk_heads, wb.num_v_heads, wb.d_k, wb.d_v,
                               wb.chunk, api.GDN_DTYPE_BF16)
        wsb = torch.empty(api.cpr2_workspace_bytes(shape_b, wb.total_tokens, wb.total_chunks,
                                                   False), dtype=torch.uint8, device="cuda")
        if trainer:
            call = lambda: api.cpr2_trainer_fwd(*d, chunk=wb.chunk, total_chunks=wb.total_chunks,
                                                workspace=wsb)
        else:
            call = lambda: api.cpr2_prefill(*d, chunk=wb.chunk, total_chunks=wb.total_chunks,
                                            workspace=wsb)
        wall_b, per_b = timed(call, 2, 1)
        mb = sum(per_b) / len(per_b)
        tb, bb, ob = cpr2_flops(wb)
        big[label] = {"kernel_ms": round(mb, 3),
                      "tokens_per_s": round(wb.total_tokens / (wall_b / 2), 1),
                      "roofline": roofline_alu(tb + bb + ob, mb)}
        del d, wsb, call
        torch.cuda.empty_cache()
    return {"workload": "two-level CPR on the trainer_fwd workload (4 x 4096 tokens, 16 heads, "
                        "d=128, C=64, bf16 q/k/v): o, the 256 chunk states (trainer) or the "
                        "final states (prefill)",
            "trainer_fwd_tokens_per_s": round(T / (wall_t / steps), 1),
            "trainer_fwd_kernel_ms": round(mt, 4),
            "prefill_tokens_per_s": round(T / (wall_p / steps), 1),
            "prefill_kernel_ms": round(mp, 4),
            "flops": {"transitions": trans, "boundary_sweep": boundary, "outputs": outputs},
            "workspace_bytes": int(need), "steps": steps, "roofline": roof,
            "hbm": hbm(cpr2_bytes(w), mt), "decode": dec, "larger_workloads": big,
            "parity": verdict(checks)}


def bench_cpr2_decode(prefix=960, nsteps=504, warmup_steps=8):
    """Two-level decode on the engine-decode workload: a two-level prefill of a chunk-aligned
    prefix (so state = boundary and the token cache is empty), then steps timed one by one;
    every 64th step rebuilds the chunk transition from the cache and sets the boundary."""
    import torch
    from bitwise_consistent_linear_amd import api
    from bitwise_consistent_linear_amd import workloads as W
    w = W.engine_decode()
    N, Hk, Hv, dk, dv, C = w.num_seqs, w.num_qk_heads, w.num_v_heads, w.d_k, w.d_v, w.chunk
    log(f"cpr2 decode: N={N}, two-level prefill of {prefix} tokens, {nsteps} decode steps")
    pre, steps = W.split_for_decode(w, prefix)
    dp = {key: up(getattr(pre, key)) for key in ("q", "k", "v", "a", "b")}
    _, fs = api.cpr2_prefill(up(pre.cu_seqlens), dp["q"], dp["k"], dp["v"], dp["a"], dp["b"],
                             chunk=C, total_chunks=pre.total_chunks)
    del dp
    torch.cuda.empty_cache()
    dec = api.Cpr2Decoder(N, Hk, Hv, dk, dv, C, torch.bfloat16, "cuda", initial_state=fs)
    del fs
    ds = {key: up(x) for key, x in steps.items()}
    rs = torch.empty_like(dec.state)
    o = torch.empty((N, Hv, dv), dtype=torch.float32, device="cuda")
    it = iter(range(ds["q"].shape[0]))

    def step():
        s = next(it)
        dec.step(ds["pos"][s], ds["q"][s], ds["k"][s], ds["v"][s], ds["a"][s], ds["b"][s],
                 o=o, resync_states=rs)

    wall, per = timed(step, nsteps, warmup_steps)
    ms = sum(per) / len(per)
    del dec, ds
    torch.cuda.empty_cache()
    # parity, after the timed run: the two-level trainer and prefill over the whole
    # 1512-token sequences; a fresh decoder from the prefix's final state must reproduce the
    # trainer's o at every later position, its chunk states at every resync and the
    # prefill's final state
    log("cpr2 decode: parity against the two-level trainer on the 1512-token sequences")
    fu = {key: up(getattr(w, key)) for key in ("cu_seqlens", "q", "k", "v", "a", "b")}
    o_full, cs_full = api.cpr2_trainer_fwd(fu["cu_seqlens"], fu["q"], fu["k"], fu["v"], fu["a"],
                                           fu["b"], chunk=C, total_chunks=w.total_chunks)
    _, fs_full = api.cpr2_prefill(fu["cu_seqlens"], fu["q"], fu["k"], fu["v"], fu["a"],
                                  fu["b"], chunk=C, total_chunks=w.total_chunks)
    del fu
    T = int(w.lengths[0])
    o_seq = o_full.view(N, T, Hv, dv)
    cs_seq = cs_full.view(N, T // C, Hv, dv, dk)
    dp = {key: up(getattr(pre, key)) for key in ("q", "k", "v", "a", "b")}
    _, fs = api.cpr2_prefill(up(pre.cu_seqlens), dp["q"], dp["k"], dp["v"], dp["a"], dp["b"],
                             chunk=C, total_chunks=pre.total_chunks)
    del dp
    dec = api.Cpr2Decoder(N, Hk, Hv, dk, dv, C, torch.bfloat16, "cuda", initial_state=fs)
    del fs
    ds = {key: up(x) for key, x in steps.items()}
    ok_o = ok_rs = True
    for s in range(T - prefix):
        dec.step(ds["pos"][s], ds["q"][s], ds["k"][s], ds["v"][s], ds["a"][s], ds["b"][s],
                 o=o, resync_states=rs)
        ok_o = ok_o and same_bits(o, o_seq[:, prefix + s])
        if (prefix + s + 1) % C == 0:
            ok_rs = ok_rs and same_bits(rs, cs_seq[:, (prefix + s + 1) // C - 1])
    checks = {f"two-level decode o == two-level trainer o ({T - prefix} steps)": ok_o,
              "two-level resyncs == two-level trainer chunk states": ok_rs,
              "two-level decode end state == two-level prefill final state":
              same_bits(dec.state, fs_full)}
    del dec, ds, o_full, cs_full, fs_full
    el = 2
    state = N * Hv * dv * dk * 4
    tok = N * (Hk * dk * el + Hv * dv * el + Hv * 8)
    # every step: the running rows (decode_step_bytes without its resync share) and the token
    # into the cache; every C steps: the cache read back, A_c and B_c written and read, the
    # boundary read and the state, boundary and resync written
    trans = N * Hv * (dk + dv) * dk * 4
    per_step = (decode_step_bytes(N, Hk, Hv, dk, dv, el, C) - state / C + tok
                + (C * tok + 2 * trans + 4 * state) / C)
    gbs = per_step / (ms * 1e-3) / 1e9
    boundary_steps = [p for s, p in enumerate(per) if (prefix + warmup_steps + s + 1) % C == 0]
    other = [p for s, p in enumerate(per) if (prefix + warmup_steps + s + 1) % C != 0]
    return {"workload": f"engine_decode workload (256 sequences, 16 q/k / 32 v heads, d=128, "
                        f"C=64), two-level prefill of {prefix} tokens, then {nsteps} steps "
                        f"({warmup_steps} untimed)",
            "us_per_step_kernel": round(ms * 1e3, 2),
            "us_per_step_wall": round(wall / nsteps * 1e6, 2),
            "us_boundary_step": round(sum(boundary_steps) / max(1, len(boundary_steps)) * 1e3, 2),
            "us_other_step": round(sum(other) / max(1, len(other)) * 1e3, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
            "algorithmic_bytes_per_step": int(per_step), "parity": verdict(checks)}


def bench_decode_after_prefill(w, prefix, nsteps, warmup_steps, label):
    """Prefill `prefix` tokens of every sequence, then time decode steps one by one."""
    import torch
    from bitwise_consistent_linear_amd import api
    from bitwise_consistent_linear_amd import workloads as W
    pre, steps = W.split_for_decode(w, prefix)
    dp = {k: up(getattr(pre, k)) for k in ("q", "k", "v", "a", "b")}
    _, state = api.prefill(up(pre.cu_seqlens), dp["q"], dp["k"], dp["v"], dp["a"], dp["b"],
                           chunk=w.chunk)
    del dp
    ds = {k: up(x) for k, x in steps.items()}
    N = w.num_seqs
    rs = torch.empty_like(state)
    o = torch.empty((N, w.num_v_heads, w.d_v), dtype=torch.float32, device="cuda")
    S = ds["q"].shape[0]
    assert warmup_steps + nsteps <= S
    it = iter(range(S))

    def step():
        s = next(it)
        api.decode_step(ds["pos"][s], ds["q"][s], ds["k"][s], ds["v"][s], ds["a"][s],
                        ds["b"][s], state, chunk=w.chunk, o=o, resync_states=rs)

    wall, per = timed(step, nsteps, warmup_steps)
    ms = sum(per) / len(per)
    # The same steps captured in one HIP graph and replayed: what an engine that captures
    # its decode loop sees, without the per-call host work of the Python binding.
    g = torch.cuda.CUDAGraph()
    first = warmup_steps
    with torch.cuda.graph(g):
        for s in range(first, first + nsteps):
            api.decode_step(ds["pos"][s], ds["q"][s], ds["k"][s], ds["v"][s], ds["a"][s],
                            ds["b"][s], state, chunk=w.chunk, o=o, resync_states=rs)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / nsteps
    del g
    nbytes = decode_step_bytes(N, w.num_qk_heads, w.num_v_heads, w.d_k, w.d_v,
                               2 if w.bf16 else 4, w.chunk)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"{label}: {nsteps} decode steps, {ms * 1e3:.1f} us/step (events per call), "
        f"{graph_us:.1f} us/step (HIP graph)")
    return {"us_per_step_kernel": round(ms * 1e3, 2),
            "us_per_step_wall": round(wall / nsteps * 1e6, 2),
            "us_per_step_hip_graph": round(graph_us, 2), "steps": nsteps,
            "warmup_steps": warmup_steps,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
            "algorithmic_bytes_per_step": int(nbytes)}


def verify_decode(w, prefix, nsteps, o_seq, cs_seq, fs_ref):
    """Parity of the decode case, after its timed run: prefill `prefix` tokens again, then
    decode `nsteps` steps one by one; every step's o must equal the trainer's o at that
    position (o_seq [N, T, Hv, dv]), every resync checkpoint the trainer's chunk state there
    (cs_seq [N, T // C, Hv, dv, dk]) and, when the steps reach the end of every sequence,
    the state the prefill of all tokens ends with (fs_ref)."""
    import torch
    from bitwise_consistent_linear_amd import api
    from bitwise_consistent_linear_amd import workloads as W
    pre, steps = W.split_for_decode(w, prefix)
    dp = {k: up(getattr(pre, k)) for k in ("q", "k", "v", "a", "b")}
    _, state = api.prefill(up(pre.cu_seqlens), dp["q"], dp["k"], dp["v"], dp["a"], dp["b"],
                           chunk=w.chunk)
    del dp
    ds = {k: up(x) for k, x in steps.items()}
    rs = torch.empty_like(state)
    o = torch.empty((w.num_seqs, w.num_v_heads, w.d_v), dtype=torch.float32, device="cuda")
    ok_o = ok_rs = True
    resyncs = 0
    for s in range(nsteps):
        api.decode_step(ds["pos"][s], ds["q"][s], ds["k"][s], ds["v"][s], ds["a"][s],
                        ds["b"][s], state, chunk=w.chunk, o=o, resync_states=rs)
        ok_o = ok_o and same_bits(o, o_seq[:, prefix + s])
        if (prefix + s + 1) % w.chunk == 0:
            resyncs += 1
            ok_rs = ok_rs and same_bits(rs, cs_seq[:, (prefix + s + 1) // w.chunk - 1])
    checks = {f"decode o == trainer o ({nsteps} steps)": ok_o,
              f"resync checkpoints == trainer chunk states ({resyncs})": ok_rs}
    if fs_ref is not None:
        checks["decode end state == prefill final state"] = same_bits(state, fs_ref)
    return checks


def copy_probe_gbs(nbytes=1 << 30, reps=5):
    """A plain device copy of nbytes (read once, written once), timed with HIP events: the
    HBM rate a streaming kernel can reach on this GPU, beside the 8 TB/s peak."""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    _, per = timed(lambda: y.copy_(x), reps, 2)
    del x, y
    ms = sorted(per)[len(per) // 2]
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


def bench_decode(verify=True, nsteps=504):
    import torch
    from bitwise_consistent_linear_amd import api
    from bitwise_consistent_linear_amd import workloads as W
    w = W.engine_decode()
    log("engine_decode: N=256, 1000-token prefill, 512 decode steps, 16/32 heads, d=128")
    r = bench_decode_after_prefill(w, 1000, nsteps, 8, "engine_decode")
    torch.cuda.empty_cache()
    if verify:
        # the trainer and prefill cases over the whole 1512-token sequences
        log("engine_decode: parity against trainer_fwd on the 1512-token sequences")
        cu, q, k, v, a, b = (up(x) for x in (w.cu_seqlens, w.q, w.k, w.v, w.a, w.b))
        o_full, cs_full = api.trainer_fwd(cu, q, k, v, a, b, chunk=w.chunk,
                                          total_chunks=w.total_chunks)
        _, fs_full = api.prefill(cu, q, k, v, a, b, chunk=w.chunk)
        del q, k, v, a, b
        N, T = w.num_seqs, int(w.lengths[0])
        checks = verify_decode(w, 1000, T - 1000,
                               o_full.view(N, T, w.num_v_heads, w.d_v),
                               cs_full.view(N, T // w.chunk, w.num_v_heads, w.d_v, w.d_k),
                               fs_full)
        r["parity"] = verdict(checks)
        del o_full, cs_full, fs_full
        torch.cuda.empty_cache()
    r["copy_probe_GBs"] = copy_probe_gbs()
    r["workload"] = ("engine_decode: 256 sequences, 16 q/k / 32 v heads, d=128, C=64, fp32 "
                     f"state in HBM, prefill 1000 tokens then {nsteps + 8} steps (8 untimed)")
    r["roofline"]["traffic"] = traffic_for("cpr_decode_engine_decode")
    return r


def bench_long(steps, scans_only=False):
    import numpy as np
    import torch
    from bitwise_consistent_linear_amd import api
    from bitwise_consistent_linear_amd import workloads as W
    w = W.long_context()
    log("long_context: T=131072, 16/32 heads, d=128")
    cu, q, k, v, a, b = (up(x) for x in (w.cu_seqlens, w.q, w.k, w.v, w.a, w.b))
    o = torch.empty((w.total_tokens, w.num_v_heads, w.d_v), dtype=torch.float32, device="cuda")
    cs = torch.empty((w.total_chunks, w.num_v_heads, w.d_v, w.d_k), dtype=torch.float32,
                     device="cuda")
    fs = torch.empty((1, w.num_v_heads, w.d_v, w.d_k), dtype=torch.float32, device="cuda")
    wall_t, per_t = timed(lambda: api.trainer_fwd(cu, q, k, v, a, b, chunk=64, o=o,
                                                  chunk_states=cs, total_chunks=w.total_chunks),
                          steps, 1)
    po = torch.empty_like(o)
    wall_p, per_p = timed(lambda: api.prefill(cu, q, k, v, a, b, chunk=64, o=po, final_state=fs),
                          steps, 1)
    del q, k, v
    torch.cuda.synchronize()
    checks = {"prefill o == trainer o": same_bits(po, o),
              "prefill final state == trainer last chunk state": same_bits(fs, cs[-1:])}
    del po
    torch.cuda.empty_cache()
    flops = flops_per_token_head(w.d_k, w.d_v) * w.total_tokens * w.num_v_heads
    mt, mp = sum(per_t) / len(per_t), sum(per_p) / len(per_p)
    if scans_only:
        return {"trainer_fwd_kernel_ms": round(mt, 3), "prefill_kernel_ms": round(mp, 3),
                "parity": verdict(checks)}
    P, S = w.extra["prefix"], w.extra["steps"]
    cut = W.Workload("long_context_decode", np.array([0, P + S], np.int32), w.q[:P + S],
                     w.k[:P + S], w.v[:P + S], w.a[:P + S], w.b[:P + S], w.chunk, w.bf16)
    dec = bench_decode_after_prefill(cut, P, S - 8, 8, "long_context decode")
    checks.update({f"after {P} tokens: {name}": ok for name, ok in verify_decode(
        cut, P, S, o.view(1, -1, w.num_v_heads, w.d_v)[:, :P + S],
        cs.view(1, -1, w.num_v_heads, w.d_v, w.d_k), None).items()})
    del o, cs
    torch.cuda.empty_cache()
    return {"workload": "long_context: 1 x 131072 tokens, 16 q/k / 32 v heads, d=128, C=64, "
                        "bf16 q/k/v, a ~ U(0.95, 1)",
            "trainer_fwd_tokens_per_s": round(w.total_tokens / (wall_t / steps), 1),
            "trainer_fwd_kernel_ms": round(mt, 3),
            "trainer_fwd_roofline": dict(roofline_alu(flops, mt),
                                         traffic=traffic_for("cpr_scan_long_context_trainer")),
            "trainer_fwd_hbm": hbm(scan_bytes(w, chunk_states=w.total_chunks), mt),
            "prefill_tokens_per_s": round(w.total_tokens / (wall_p / steps), 1),
            "prefill_kernel_ms": round(mp, 3),
            "prefill_roofline": dict(roofline_alu(flops, mp),
                                     traffic=traffic_for("cpr_scan_long_context_prefill")),
            "prefill_hbm": hbm(scan_bytes(w, final_states=1), mp),
            "decode_after_65536": dec, "parity": verdict(checks)}


def cpu_baseline(w, gpu_outputs):
    """The CPU oracle on the whole trainer_fwd workload (all outputs), on the host's cores,
    and whether its outputs equal the GPU's trainer_fwd outputs bit for bit."""
    import numpy as np
    from oracle import oracle as O
    threads = min(16, O.default_threads())
    t0 = time.perf_counter()
    ro, rcs, _ = O.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=w.chunk,
                        want_chunk_states=True, nthreads=threads)
    dt = time.perf_counter() - t0
    go, gcs = gpu_outputs
    same = (np.array_equal(np.ascontiguousarray(go).view(np.uint32), ro.view(np.uint32))
            and np.array_equal(np.ascontiguousarray(gcs).view(np.uint32), rcs.view(np.uint32)))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         "")
    except OSError:
        pass
    return {"value": round(w.total_tokens / dt, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "affinity_cores": O.default_threads(), "cpu_model": model,
            "sample": f"the whole trainer_fwd workload (4 x 4096 tokens, 16 heads, o and "
                      f"chunk states), {dt:.2f} s on {threads} threads",
            "bitwise_equal_to_gpu_trainer_fwd": bool(same)}


TRACE_TITLES = {
    "main": ("cpr_scan_trainer_fwd", "trainer_fwd: 4 x 4096 tokens, 16 heads, d_k = d_v = 128, "
             "C = 64, bf16 q/k/v"),
    "prefill": ("cpr_scan_engine_prefill", "engine_prefill: 64 varlen sequences, 262144 tokens, "
                "16 q/k / 32 v heads, d = 128, bf16 q/k/v"),
    "decode": ("cpr_decode_engine_decode", "engine_decode: 256 sequences, 16 q/k / 32 v heads, "
               "d = 128, C = 64, 1000-token prefill then 512 steps"),
    "long": ("cpr_scan_long_context", "long_context: 1 x 131072 tokens, 16 q/k / 32 v heads, "
             "d = 128, C = 64: trainer_fwd, prefill, prefill of 65536 then 256 decode steps"),
    "bwd": ("cpr_bwd_trainer", "trainer_bwd on the trainer_fwd workload"),
    "cpr2": ("cpr2_two_level", "two-level CPR: trainer, prefill and decode"),
    "linear": ("linear_leaf_16384x4096x4096", "linear region: 16384 x 4096 x 4096, bf16 in, "
               "binary32 out"),
}
TRACE_COMMAND = ("export TMPDIR=/tmp; cd /tmp && rocprofv3 --kernel-trace --stats --output-format "
                 "csv -d $R/gpurun_out/trace_{case} -o {case} -- python3 $R/bench.py --cases "
                 "{case} --no-cpu-baseline --steps 20")


def write_trace_summary(stats_csv, case, bench_json=None):
    """profiles/<name>_kernel_trace.md from a rocprofv3 --kernel-trace --stats run of
    `bench.py --cases <case>`: the command, each kernel's calls and average duration, and,
    when the JSON line of a bench run in the same lease is given, the bench's own event
    timings beside them."""
    import csv
    name, title = TRACE_TITLES[case]
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# {title} (rocprofv3 kernel-trace stats)", "",
             "Command (one MI355X, repository root as R):", "", "```",
             TRACE_COMMAND.format(case=case), "```", "",
             "| kernel | calls | average ns | min ns | max ns | % |", "|---|---|---|---|---|---|"]
    for r in rows[:12]:
        kname = r["Name"] if len(r["Name"]) <= 110 else r["Name"][:100] + " ..."
        lines.append(f"| `{kname}` | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                     f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f} | "
                     f"{float(r['Percentage']):.2f} |")
    if bench_json:
        with open(bench_json) as f:
            line = [ln for ln in f.read().splitlines() if ln.startswith("{")][-1]
        b = json.loads(line)
        lines += ["", "The bench run in the same lease (HIP events on the launching stream):", ""]
        lines.append(f"- trainer_fwd: {b['kernel_ms']} ms per call, roofline "
                     f"{json.dumps(b['roofline'])}, parity {b['parity']['bitwise_exact']}")
        if b.get("valu_probe"):
            lines.append(f"- shader clock (probe): {b['valu_probe']['shader_clock_GHz']} GHz")
        for cname, c in (b.get("cases") or {}).items():
            keep = {k: v for k, v in c.items()
                    if k.endswith("_ms") or k.startswith("us_") or k.endswith("roofline")}
            lines.append(f"- {cname}: {json.dumps(keep)}; parity "
                         f"{c.get('parity', {}).get('bitwise_exact')}")
    path = os.path.join(ROOT, "profiles", f"{name}_kernel_trace.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cases",
                    choices=["all", "main", "bwd", "prefill", "decode", "long", "linear", "cpr2",
                             "traffic"],
                    default="all",
                    help="all: every case; main: trainer_fwd only; bwd / prefill / decode / long "
                         "/ linear / cpr2: trainer_fwd and the backward / the engine_prefill call "
                         "/ the engine_decode steps / the long-context calls / the linear region "
                         "/ the two-level reading (for profiling); traffic: a few calls of every "
                         "one-level scan, the decode step, the backward, the two-level "
                         "trainer and the linear region (for the counter runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (untimed), the known-size "
                         "reference that calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/*_traffic.json from two rocprofv3 counter CSVs and "
                         "exit (no GPU needed)")
    ap.add_argument("--trace-summary", nargs=2, metavar=("STATS_CSV", "CASE"),
                    help="write profiles/<kernel>_kernel_trace.md from the kernel_stats.csv of "
                         "a traced `bench.py --cases CASE` run and exit (no GPU needed)")
    ap.add_argument("--bench-json", help="with --trace-summary: the JSON line of a bench run "
                                         "in the same lease, quoted beside the trace")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic(*args.traffic_from)
        return
    if args.trace_summary:
        write_trace_summary(*args.trace_summary, bench_json=args.bench_json)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path. Every state row "
              "evolves on its own, so sequences and value heads would split across GPUs with "
              "no exchange and no change of bits.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from bitwise_consistent_linear_amd import api
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    api.lib()
    log(f"device: {torch.cuda.get_device_name(0)}")

    if args.copy_probe:
        x = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        del x, y
    w, wall, kernel_ms, flops, nbytes, par, outputs = bench_trainer(args.steps, args.warmup)
    ms_per_step = wall / args.steps * 1e3
    roof = roofline_alu(flops, kernel_ms)
    traffic = traffic_for("cpr_scan_trainer_fwd")
    roof["traffic"] = traffic
    log(f"trainer_fwd: {ms_per_step:.3f} ms/step, kernel {kernel_ms:.3f} ms, "
        f"{roof['achieved']} TFLOP/s, parity {par['bitwise_exact']}")
    torch.cuda.empty_cache()
    probe = valu_probe() if args.cases != "traffic" else None
    out = {
        "metric": METRIC,
        "value": round(w.total_tokens / (wall / args.steps), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "trainer_fwd: 4 sequences x 4096 tokens, 16 q/k = 16 v heads, "
                               "d_k=d_v=128, C=64, bf16 q/k/v, fp32 a/b/state/o; writes o and "
                               "the 256 chunk-boundary states",
                   "global_batch": 4, "seq_len": 4096, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "hbm": hbm(nbytes, kernel_ms),
        "parity": par,
        "kernel_ms": round(kernel_ms, 4),
        "valu_probe": probe,
        "contract_identity": api.contract_identity(64, 128).hex(),
    }
    steps4 = max(3, args.steps // 4)
    runners = {
        "trainer_bwd": lambda: bench_trainer_bwd(steps4, 1, kernel_ms),
        "engine_prefill": lambda: bench_prefill(steps4, 1),
        "engine_decode": lambda: bench_decode(),
        "long_context": lambda: bench_long(max(2, args.steps // 10)),
        "linear": lambda: bench_linear(steps4, 1),
        "two_level": lambda: bench_cpr2(steps4, 1),
    }
    chosen = {"all": list(runners), "main": [], "bwd": ["trainer_bwd"],
              "prefill": ["engine_prefill"], "decode": ["engine_decode"], "long": ["long_context"],
              "linear": ["linear"], "cpr2": ["two_level"]}
    if args.cases == "traffic":
        runners.update({
            "trainer_bwd": lambda: bench_trainer_bwd(3, 1, kernel_ms, verify=False),
            "two_level": lambda: bench_cpr2(3, 1, trainer_only=True),
            "engine_prefill": lambda: bench_prefill(2, 1),
            "engine_decode": lambda: bench_decode(verify=False, nsteps=16),
            "long_context": lambda: bench_long(1, scans_only=True),
            "linear": lambda: bench_linear(2, 1),
        })
        names = ["trainer_bwd", "two_level", "engine_prefill", "engine_decode", "long_context",
                 "linear"]
    else:
        names = chosen[args.cases]
    if names:
        out["cases"] = {}
        for name in names:
            out["cases"][name] = runners[name]()
            torch.cuda.empty_cache()
    def verdicts(node):  # every parity verdict in the line, nested ones included
        if isinstance(node, dict):
            if "bitwise_exact" in node and "checks" in node:
                yield node["bitwise_exact"]
            for child in node.values():
                yield from verdicts(child)
    out["parity_all_bitwise_exact"] = all(verdicts(out))
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on the trainer_fwd workload")
        out["cpu_baseline"] = cpu_baseline(w, outputs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
