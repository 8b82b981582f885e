"""GPU parity: the HIP kernels, called through the C ABI, against the CPU oracle and against
each other, bit for bit.

Small cases (ragged lengths, empty sequences, GQA, every d_k, f32 and bf16 storage, ragged
d_v, initial states, every lanes-per-row value) are compared element by element with the
oracle. The five workload configurations run at full size in the launch configuration
that bench.py times: the three cases are compared with each other over every output on
the device, and with the oracle on sampled (sequence, head) pairs that it computes alone.
"""

import zlib

import numpy as np
import pytest
import torch

from bitwise_consistent_linear_amd import api
from bitwise_consistent_linear_amd import workloads as W
from gpu_util import (DEV, LANES, assert_bits, assert_dev_equal, decode_steps, lanes, log,
                      rows_per_group, scan_threads, up, up_steps, up_workload)
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def run_trainer(w, d, s0=None, total_chunks=None):
    return api.trainer_fwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], chunk=w.chunk,
                           initial_state=s0, total_chunks=w.total_chunks if total_chunks is None
                           else total_chunks)


def run_prefill(w, d, s0=None):
    return api.prefill(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], chunk=w.chunk,
                       initial_state=s0)


# ----------------------------------------------------------------------------- tiny

def test_tiny_three_cases_match_oracle():
    w = W.tiny()
    log("tiny: N=1 T=64 H=2 d=16 C=16 f32")
    d = up_workload(w)
    ro, rcs, rfs = O.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=w.chunk,
                          want_chunk_states=True, want_final_state=True)
    for L in LANES:
        with lanes(L):
            o, cs = run_trainer(w, d)
            po, fs = run_prefill(w, d)
            state = torch.zeros_like(fs)
            outs, resyncs = [], []
            pos = torch.arange(64, dtype=torch.int32, device=DEV).view(64, 1)
            for t in range(64):
                rs = torch.zeros_like(state)
                outs.append(api.decode_step(pos[t], d["q"][t:t + 1], d["k"][t:t + 1],
                                            d["v"][t:t + 1], d["a"][t:t + 1], d["b"][t:t + 1],
                                            state, chunk=w.chunk, resync_states=rs))
                if (t + 1) % w.chunk == 0:
                    resyncs.append(rs)
                else:
                    assert not rs.any(), f"resync written off-boundary at t={t}"
            torch.cuda.synchronize()
        assert_bits(o, ro, f"L={L} trainer o")
        assert_bits(cs, rcs, f"L={L} trainer chunk states")
        assert_bits(po, ro, f"L={L} prefill o")
        assert_bits(fs, rfs, f"L={L} prefill final state")
        assert_bits(torch.cat(outs), ro, f"L={L} decode o")
        assert_bits(state, rfs, f"L={L} decode state")
        assert_bits(torch.cat(resyncs), rcs, f"L={L} decode resync")


# ------------------------------------------------------------------------- small cases

SMALL = [
    # name, lengths, Hk, Hv, d_k, d_v, chunk, bf16, with_s0
    ("d16_ragged_f32", [5, 0, 37, 16, 1], 1, 2, 16, 16, 16, False, True),
    ("d32_gqa2_bf16", [23, 64, 17], 2, 4, 32, 32, 32, True, False),
    ("d64_gqa4_bf16_s0", [100, 3, 48], 1, 4, 64, 64, 16, True, True),
    ("d128_bf16_c64", [130, 64, 0, 77], 2, 2, 128, 128, 64, True, True),
    ("d128_f32_c256", [300, 17], 1, 2, 128, 128, 256, False, True),
    ("d64_dv40_ragged_rows", [33, 50], 1, 2, 64, 40, 16, True, True),
    ("d128_dv72", [45, 19], 2, 4, 128, 72, 32, False, False),
    ("d16_dv256", [20], 1, 1, 16, 256, 16, True, True),
    ("d128_empty_batch_of_zero_lengths", [0, 0, 0], 1, 2, 128, 128, 64, True, True),
    # few rows and bf16: at 16 lanes per row the scan stages 64 tokens at a time, and chunk
    # boundaries fall on every second or fourth stage end
    ("d128_bf16_c128_long_stages", [300, 129, 64], 1, 2, 128, 128, 128, True, True),
    ("d128_bf16_c256_long_stages", [520, 255], 1, 1, 128, 128, 256, True, False),
    # the largest admitted rows (d_v = 1024 at d_k = 128), and the largest admitted token
    # width: Hv * max(d_k, d_v) = 2^20, the bound of the kernels' 32-bit in-stage offsets
    ("d128_dv1024_max_rows", [40, 7], 1, 1, 128, 1024, 64, True, True),
    ("max_head_width", [20, 3], 1024, 1024, 16, 1024, 16, True, False),
]


def small_workload(name, lengths, Hk, Hv, dk, dv, chunk, bf16, with_s0):
    seed = zlib.crc32(name.encode()) % 1000
    w = W.make_packed(name, lengths, Hk=Hk, Hv=Hv, d=dk, chunk=chunk, bf16=bf16, seed=500 + seed)
    if dv != dk:  # replace v with a [T, Hv, dv] draw of the same recipe
        w2 = W.make_packed(name, lengths, Hk=Hv, Hv=Hv, d=dv, chunk=chunk, bf16=bf16,
                           seed=900 + seed)
        w.v = w2.v
    s0 = None
    if with_s0:
        g = np.random.default_rng(seed)
        s0 = (0.25 * g.standard_normal((len(lengths), Hv, dv, dk))).astype(np.float32)
    return w, s0


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases_match_oracle(case):
    w, s0 = small_workload(*case)
    log(f"small: {case}")
    ro, rcs, rfs = O.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=w.chunk,
                          initial_state=s0, want_chunk_states=True, want_final_state=True)
    d = up_workload(w)
    ds0 = None if s0 is None else up(s0)
    for L in LANES:
        with lanes(L):
            o, cs = run_trainer(w, d, ds0)
            po, fs = run_prefill(w, d, ds0)
            torch.cuda.synchronize()
        assert_bits(o, ro, f"{case[0]} L={L} trainer o")
        assert_bits(cs, rcs, f"{case[0]} L={L} trainer chunk states")
        assert_bits(po, ro, f"{case[0]} L={L} prefill o")
        assert_bits(fs, rfs, f"{case[0]} L={L} prefill final")
    # two rows per group of 4 lanes (128-row workgroups)
    with lanes(4), rows_per_group(2):
        o, cs = run_trainer(w, d, ds0)
        po, fs = run_prefill(w, d, ds0)
        torch.cuda.synchronize()
    assert_bits(o, ro, f"{case[0]} L=4 row pairs trainer o")
    assert_bits(cs, rcs, f"{case[0]} L=4 row pairs trainer chunk states")
    assert_bits(po, ro, f"{case[0]} L=4 row pairs prefill o")
    assert_bits(fs, rfs, f"{case[0]} L=4 row pairs prefill final")


# 512-thread workgroups (32 rows, 64-token stages, a one-stage o buffer written back per
# wave) forced on small bf16 batches whose d_v is a multiple of 32: ragged and empty
# sequences, last stages of every length, GQA, C = 64 and 128, an initial state
SMALL_512 = [
    ("d128_c64_ragged_stages", [0, 1, 63, 64, 65, 200, 130], 2, 4, 128, 128, 64, True, True),
    ("d64_dv96_c128_gqa", [129, 300, 7], 1, 4, 64, 96, 128, True, False),
    ("d32_dv32_c64", [1, 127, 64], 1, 1, 32, 32, 64, True, True),
]


@pytest.mark.parametrize("case", SMALL_512, ids=[c[0] for c in SMALL_512])
def test_small_cases_512_threads_match_oracle(case):
    w, s0 = small_workload(*case)
    log(f"small, 512-thread scan: {case}")
    ro, rcs, rfs = O.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=w.chunk,
                          initial_state=s0, want_chunk_states=True, want_final_state=True)
    d = up_workload(w)
    ds0 = None if s0 is None else up(s0)
    with lanes(16), scan_threads(512):
        o, cs = run_trainer(w, d, ds0)
        po, fs = run_prefill(w, d, ds0)
        torch.cuda.synchronize()
    assert_bits(o, ro, f"{case[0]} trainer o")
    assert_bits(cs, rcs, f"{case[0]} trainer chunk states")
    assert_bits(po, ro, f"{case[0]} prefill o")
    assert_bits(fs, rfs, f"{case[0]} prefill final")


@pytest.mark.parametrize("L", LANES + (32,))
def test_decode_matches_oracle_and_trainer(L):
    # equal-length batch: prefix by prefill, then decode steps across several boundaries
    w = W.make_packed("dec", [90] * 3, Hk=2, Hv=4, d=64, chunk=16, bf16=True, seed=77)
    g = np.random.default_rng(7)
    s0 = (0.25 * g.standard_normal((3, 4, 64, 64))).astype(np.float32)
    log(f"decode small L={L}")
    ro, rcs, rfs = O.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=16, initial_state=s0,
                          want_chunk_states=True, want_final_state=True)
    pre, steps = W.split_for_decode(w, 21)
    dp = up_workload(pre)
    with lanes(L):
        _, state = run_prefill(pre, dp, up(s0))
        dsteps = up_steps(steps)
        ro_seq = ro.reshape(3, 90, 4, 64)
        rcs_seq = rcs.reshape(3, 5, 4, 64, 64)
        for s, o, rs in decode_steps(dsteps, state, 16):
            assert_bits(o, ro_seq[:, 21 + s], f"decode o step {s}")
            if (21 + s + 1) % 16 == 0:
                assert_bits(rs, rcs_seq[:, (21 + s + 1) // 16 - 1], f"resync step {s}")
    assert_bits(state, rfs, "decode final state")


@pytest.mark.parametrize("dk,dv,bf16", [(32, 32, False), (128, 40, True), (64, 64, False)])
def test_decode_32_lanes_per_row(dk, dv, bf16):
    # a row on 32 lanes (each leaf's chain handed from one lane to the next) for every d_k
    # that admits it, binary32 and bf16 inputs, a d_v that ends part-way through a workgroup
    w = W.make_packed("dec32", [40] * 2, Hk=1, Hv=2, d=dk, chunk=16, bf16=bf16, seed=79)
    if dv != dk:
        w.v = W.make_packed("dec32", [40] * 2, Hk=2, Hv=2, d=dv, chunk=16, bf16=bf16,
                            seed=80).v
    g = np.random.default_rng(9)
    s0 = (0.25 * g.standard_normal((2, 2, dv, dk))).astype(np.float32)
    log(f"decode 32 lanes per row: d_k={dk} d_v={dv} bf16={bf16}")
    ro, rcs, rfs = O.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=16, initial_state=s0,
                          want_chunk_states=True, want_final_state=True)
    pre, steps = W.split_for_decode(w, 5)
    dp = up_workload(pre)
    with lanes(32):
        _, state = run_prefill(pre, dp, up(s0))
        dsteps = up_steps(steps)
        ro_seq = ro.reshape(2, 40, 2, dv)
        rcs_seq = rcs.reshape(2, 2, 2, dv, dk)
        for s, o, rs in decode_steps(dsteps, state, 16):
            assert_bits(o, ro_seq[:, 5 + s], f"decode o step {s}")
            if (5 + s + 1) % 16 == 0:
                assert_bits(rs, rcs_seq[:, (5 + s + 1) // 16 - 1], f"resync step {s}")
    assert_bits(state, rfs, "decode final state")


def test_decode_idle_slots_untouched():
    w = W.make_packed("idle", [4] * 3, Hk=1, Hv=2, d=32, chunk=16, bf16=False, seed=78)
    pre, steps = W.split_for_decode(w, 3)
    g = np.random.default_rng(8)
    s0 = g.standard_normal((3, 2, 32, 32)).astype(np.float32)
    state = up(s0)
    pos = up(np.array([-1, 15, -7], np.int32))
    o = torch.full((3, 2, 32), 7.0, device=DEV)
    rs = torch.full_like(state, 9.0)
    dst = up_steps(steps)
    api.decode_step(pos, dst["q"][0], dst["k"][0], dst["v"][0], dst["a"][0], dst["b"][0], state,
                    chunk=16, o=o, resync_states=rs)
    st = s0.copy()
    ro, rrs = O.decode_step(np.array([-1, 15, -7], np.int32), steps["q"][0], steps["k"][0],
                            steps["v"][0], steps["a"][0], steps["b"][0], st, chunk=16)
    assert_bits(state, st, "states after a step with idle slots")
    assert_bits(o[1], ro[1], "active slot o")
    assert torch.all(o[0] == 7.0) and torch.all(o[2] == 7.0), "idle slot o written"
    assert_bits(rs[1], rrs[1], "active slot resync")
    assert torch.all(rs[0] == 9.0) and torch.all(rs[2] == 9.0), "idle slot resync written"


def test_prefill_in_place_state():
    w, s0 = small_workload("inplace", [40, 9], 1, 2, 64, 64, 16, True, True)
    d = up_workload(w)
    buf = up(s0)
    api.prefill(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], chunk=16, initial_state=buf,
                final_state=buf)
    _, _, rfs = O.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=16, initial_state=s0,
                       want_o=False, want_final_state=True)
    assert_bits(buf, rfs, "in-place prefill")


def test_refused_call_leaves_outputs_untouched():
    w = W.tiny()
    d = up_workload(w)
    o = torch.full((64, 2, 16), 3.0, device=DEV)
    with pytest.raises(api.GdnError) as e:
        api.trainer_fwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], chunk=16, o=o,
                        identity=bytes(32))
    assert e.value.status == api.GDN_E_IDENTITY
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)


def test_repeat_runs_identical():
    w, s0 = small_workload("repeat", [700, 333, 1000], 2, 4, 128, 128, 64, True, True)
    d = up_workload(w)
    ds0 = up(s0)
    first = run_trainer(w, d, ds0)
    for _ in range(4):
        again = run_trainer(w, d, ds0)
        assert_dev_equal(again[0], first[0], "repeat o")
        assert_dev_equal(again[1], first[1], "repeat chunk states")


# ------------------------------------------------------------------- full-size configs

def sampled_oracle(w, pairs, o_dev, cs_dev=None, fs_dev=None, s0=None):
    """Oracle on selected (n, h) pairs only, compared with the device outputs."""
    res = O.scan_pairs(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, pairs, chunk=w.chunk,
                       initial_state=s0)
    coff = np.concatenate([[0], np.cumsum(w.lengths // w.chunk)])
    for (n, h), r in zip(pairs, res):
        sl = slice(int(w.cu_seqlens[n]), int(w.cu_seqlens[n + 1]))
        assert_bits(o_dev[sl, h], r["o"], f"{w.name} oracle o (n={n}, h={h})")
        if cs_dev is not None:
            assert_bits(cs_dev[coff[n]:coff[n + 1], h], r["chunk_states"],
                        f"{w.name} oracle chunk states (n={n}, h={h})")
        if fs_dev is not None:
            assert_bits(fs_dev[n, h], r["final_state"], f"{w.name} oracle final (n={n}, h={h})")


def test_config_trainer_fwd():
    w = W.trainer_fwd()
    log("trainer_fwd: N=4 T=4096 H=16 d=128 C=64 bf16")
    d = up_workload(w)
    o, cs = run_trainer(w, d)
    po, fs = run_prefill(w, d)
    torch.cuda.synchronize()
    assert_dev_equal(po, o, "trainer vs prefill o")
    last = cs.view(4, 64, 16, 128, 128)[:, -1]
    assert_dev_equal(fs, last, "prefill final vs last chunk state")
    for L, R in ((8, 1), (4, 1), (4, 2)):
        with lanes(L), rows_per_group(R):
            o2, cs2 = run_trainer(w, d)
        assert_dev_equal(o2, o, f"L={L} R={R} vs L=16 o")
        assert_dev_equal(cs2, cs, f"L={L} R={R} vs L=16 chunk states")
    # this shape runs in 512-thread workgroups with 64-token stages; 256 threads and
    # 32-token stages give the same bits
    with scan_threads(256):
        o3, cs3 = run_trainer(w, d)
        po3, fs3 = run_prefill(w, d)
    assert_dev_equal(o3, o, "256 vs 512 threads o")
    assert_dev_equal(cs3, cs, "256 vs 512 threads chunk states")
    assert_dev_equal(po3, po, "256 vs 512 threads prefill o")
    assert_dev_equal(fs3, fs, "256 vs 512 threads final states")
    sampled_oracle(w, [(0, 0), (3, 15), (1, 6)], o, cs, fs)


def test_config_engine_prefill():
    w = W.engine_prefill()
    L = w.lengths
    log(f"engine_prefill: N=64 varlen {L.min()}..{L.max()} sum {L.sum()} Hk=16 Hv=32 d=128")
    d = up_workload(w)
    po, fs = run_prefill(w, d)
    o, cs = run_trainer(w, d)
    torch.cuda.synchronize()
    assert_dev_equal(o, po, "trainer vs prefill o")
    # this shape runs two rows per group of 4 lanes; one row per group gives the same bits
    with rows_per_group(1):
        po1, fs1 = run_prefill(w, d)
    assert_dev_equal(po1, po, "one vs two rows per group prefill o")
    assert_dev_equal(fs1, fs, "one vs two rows per group final states")
    longest, shortest = int(np.argmax(L)), int(np.argmin(L))
    sampled_oracle(w, [(longest, 31), (shortest, 0), (7, 13)], po, cs, fs)


def test_config_engine_decode():
    w = W.engine_decode()
    prefix, nsteps = w.extra["prefix"], w.extra["steps"]
    log(f"engine_decode: N=256 prefix {prefix} + {nsteps} decode steps, Hk=16 Hv=32 d=128")
    d = up_workload(w)
    o_full, cs_full = run_trainer(w, d)
    _, fs_full = run_prefill(w, d)
    pre, steps = W.split_for_decode(w, prefix)
    del d
    _, state = run_prefill(pre, up_workload(pre))
    dst = up_steps(steps)
    N, T = w.num_seqs, prefix + nsteps
    o_seq = o_full.view(N, T, 32, 128)
    cs_seq = cs_full.view(N, T // 64, 32, 128, 128)
    for s, o, rs in decode_steps(dst, state, 64):
        assert_dev_equal(o, o_seq[:, prefix + s], f"decode step {s} o vs trainer")
        if (prefix + s + 1) % 64 == 0:
            assert_dev_equal(rs, cs_seq[:, (prefix + s + 1) // 64 - 1], f"resync step {s}")
    assert_dev_equal(state, fs_full, "decode end state vs prefill of all tokens")
    sampled_oracle(w, [(0, 0), (255, 31), (100, 17)], o_full, cs_full, fs_full)


def test_config_long_context():
    w = W.long_context()
    prefix, nsteps = w.extra["prefix"], w.extra["steps"]
    log(f"long_context: T=131072 Hk=16 Hv=32 d=128; decode {nsteps} after {prefix}")
    d = up_workload(w)
    o, cs = run_trainer(w, d)
    po, fs = run_prefill(w, d)
    torch.cuda.synchronize()
    assert_dev_equal(po, o, "trainer vs prefill o")
    assert_dev_equal(fs, cs[-1:], "prefill final vs last chunk state")
    # prefill the prefix, then decode: must continue the same bits
    cut = W.Workload("long_prefix", np.array([0, prefix], np.int32), w.q[:prefix],
                     w.k[:prefix], w.v[:prefix], w.a[:prefix], w.b[:prefix], 64, True)
    _, state = run_prefill(cut, {k: v[:prefix] if k != "cu" else up(cut.cu_seqlens)
                                 for k, v in d.items()})
    rs = torch.empty_like(state)
    for s in range(nsteps):
        t = prefix + s
        pos = torch.full((1,), t, dtype=torch.int32, device=DEV)
        od = api.decode_step(pos, d["q"][t:t + 1], d["k"][t:t + 1], d["v"][t:t + 1],
                             d["a"][t:t + 1], d["b"][t:t + 1], state, chunk=64,
                             resync_states=rs)
        assert_dev_equal(od, o[t:t + 1], f"long decode step {s}")
        if (t + 1) % 64 == 0:
            assert_dev_equal(rs, cs[(t + 1) // 64 - 1:(t + 1) // 64], f"long resync step {s}")
    sampled_oracle(w, [(0, 0), (0, 31)], o, cs, fs)


# ------------------------------------------------------------------ more edge cases

def test_many_sequences_unranked_path():
    # more than 1024 sequences: workgroups take sequences in natural order (no length rank)
    g = np.random.default_rng(21)
    lengths = g.integers(0, 40, 1100)
    w = W.make_packed("many", lengths, Hk=1, Hv=2, d=32, chunk=16, bf16=True, seed=21)
    log(f"many sequences: N={w.num_seqs} T={w.total_tokens}")
    ro, rcs, rfs = O.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=16,
                          want_chunk_states=True, want_final_state=True)
    d = up_workload(w)
    for L in LANES:
        with lanes(L):
            o, cs = run_trainer(w, d)
            po, fs = run_prefill(w, d)
        assert_bits(o, ro, f"many L={L} trainer o")
        assert_bits(cs, rcs, f"many L={L} chunk states")
        assert_bits(po, ro, f"many L={L} prefill o")
        assert_bits(fs, rfs, f"many L={L} final")


def test_subnormal_states_kept():
    # a tiny decay drives the state into the binary32 subnormal range; the contract keeps
    # denormals, so GPU and oracle must agree bit for bit there too
    w, s0 = small_workload("subnormal", [48, 20], 1, 2, 64, 64, 16, False, True)
    w.a[:] = np.float32(2.0 ** -20)
    w.b[:] = np.float32(2.0 ** -60)
    w.v *= np.float32(2.0 ** -70)
    ro, rcs, rfs = O.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=16, initial_state=s0,
                          want_chunk_states=True, want_final_state=True)
    tiny = np.abs(rfs[rfs != 0])
    assert tiny.size and (tiny < np.float32(2.0 ** -126)).mean() > 0.5, "case must reach subnormals"
    d = up_workload(w)
    for L in LANES:
        with lanes(L):
            o, cs = run_trainer(w, d, up(s0))
            po, fs = run_prefill(w, d, up(s0))
        assert_bits(o, ro, f"subnormal L={L} o")
        assert_bits(cs, rcs, f"subnormal L={L} chunk states")
        assert_bits(fs, rfs, f"subnormal L={L} final")


def test_onehot_closed_form_on_gpu():
    # exact arithmetic: one-hot k and q, a in {1, 1/2}, b in {0, 1}, small-integer v and S0
    import oracle_pins
    cu, q, k, v, a, b, s0, kap, rho = oracle_pins.onehot_case(T=40, Hk=2, Hv=4, d=32, seed=9)
    ro, rcs, rfs = O.scan(cu, q, k, v, a, b, chunk=16, initial_state=s0,
                          want_chunk_states=True, want_final_state=True)
    dcu, dq, dk, dv, da, db = map(up, (cu, q, k, v, a, b))
    for L in LANES:
        with lanes(L):
            o, cs = api.trainer_fwd(dcu, dq, dk, dv, da, db, chunk=16, initial_state=up(s0))
        assert_bits(o, ro, f"one-hot L={L} o")
        assert_bits(cs, rcs, f"one-hot L={L} chunk states")


@pytest.mark.parametrize("chunk", [16, 128, 256])
def test_config_trainer_fwd_other_chunks(chunk):
    # C changes only which states are emitted: o is the same bits for every C, and every
    # emitted state equals the C=64 run's state at the same token
    w = W.trainer_fwd()
    d = up_workload(w)
    o64, cs64 = run_trainer(w, d)
    w.chunk = chunk
    o, cs = run_trainer(w, d)
    assert_dev_equal(o, o64, f"C={chunk} vs C=64 o")
    per = 4096 // chunk
    a = cs.view(4, per, 16, 128, 128)
    b = cs64.view(4, 64, 16, 128, 128)
    if chunk < 64:
        assert_dev_equal(a[:, 64 // chunk - 1::64 // chunk].contiguous(), b, "boundary states")
    else:
        assert_dev_equal(a, b[:, chunk // 64 - 1::chunk // 64].contiguous(), "boundary states")
    sampled_oracle(w, [(2, 9)], o, cs)


def test_decode_steps_in_hip_graph_match_eager():
    # Decode steps captured once into a HIP graph (the library only launches kernels on the
    # caller's stream) and replayed: every replay, run after eager work and a sync, must
    # give the bits of the same steps run eagerly.
    w = W.make_packed("graph", [40] * 6, Hk=2, Hv=4, d=64, chunk=16, bf16=True, seed=31)
    pre, steps = W.split_for_decode(w, 24)
    dst = up_steps(steps)
    _, s_start = run_prefill(pre, up_workload(pre))
    S = dst["q"].shape[0]
    # eager reference
    st = s_start.clone()
    ref_o, ref_rs = [], []
    for s, o, rs in decode_steps(dst, st, 16):
        ref_o.append(o.clone())
        ref_rs.append(rs.clone())
    ref_state = st.clone()
    # capture
    state = s_start.clone()
    outs = [torch.empty_like(ref_o[0]) for _ in range(S)]
    rss = [torch.empty_like(state) for _ in range(S)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(S):
            api.decode_step(dst["pos"][s], dst["q"][s], dst["k"][s], dst["v"][s], dst["a"][s],
                            dst["b"][s], state, chunk=16, o=outs[s], resync_states=rss[s])
    for replay in range(3):
        junk = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        state.copy_(s_start)
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        del junk
        for s in range(S):
            assert_dev_equal(outs[s], ref_o[s], f"replay {replay} step {s} o")
            if (24 + s + 1) % 16 == 0:
                assert_dev_equal(rss[s], ref_rs[s], f"replay {replay} step {s} resync")
        assert_dev_equal(state, ref_state, f"replay {replay} final state")
