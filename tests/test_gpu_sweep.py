"""GPU parity over a seeded sweep of random small shapes, bit for bit against the oracle.

The hand-picked cases of the other GPU tests each pin one feature; here one seeded draw
mixes them: every admitted d_k and C, GQA groups, ragged d_v (row blocks that end part-way
and d_v below a wave's rows), empty and ragged sequences whose lengths end anywhere
relative to C and to the scan's stages, f32 and bf16 storage, initial states and
dL/dS_final present or absent, and a launch configuration (lanes per row, scan workgroup
size, rows per group of lanes, backward schedule) drawn with them. The forward's trainer output, chunk states,
prefill output and final state and the backward's six gradients are compared element by
element with the oracle on the same inputs. The draw is fixed by its seed, so a failure
names a case that reproduces.
"""

import numpy as np
import pytest
import torch

from bitwise_consistent_linear_amd import api
from bitwise_consistent_linear_amd import workloads as W
from gpu_util import (assert_bits, lanes, log, rows_per_group, scan_threads, schedule, up,
                      up_workload)
from oracle import oracle as O

SWEEP_SEED = 20261203
SWEEP_CASES = 96


def draw_cases(seed=SWEEP_SEED, n=SWEEP_CASES):
    """n case tuples (name, lengths, Hk, Hv, d_k, d_v, chunk, bf16, with_s0, with_dsf, L,
    threads, bwd schedule, data seed, rows per group), sized so that the oracle's backward
    of the largest stays near a second. Every fourth case is drawn where 512-thread scan
    workgroups are admitted (16 lanes per row, bf16, d_v a multiple of 32) and asks for
    them; every other case is run with two rows per group of lanes where it has 4 lanes per
    row (the row-pair count takes no draw, so the other fields are as drawn before)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        wide = i % 4 == 3
        dk = int(rng.choice([16, 32, 64, 128]))
        chunk = int(rng.choice([16, 32, 64, 128, 256]))
        Hk = int(rng.choice([1, 2]))
        Hv = min(Hk * int(rng.choice([1, 2, 4])), 4)
        if wide:
            dv = 32 * int(rng.integers(1, 5))
        else:
            dv = dk if rng.random() < 0.5 else int(rng.integers(1, 161))
        nseq = int(rng.integers(1, 7))
        lengths = [0 if rng.random() < 0.15 else int(rng.integers(1, 3 * chunk + 10))
                   for _ in range(nseq)]
        bf16 = True if wide else bool(rng.random() < 0.6)
        with_s0 = bool(rng.random() < 0.5)
        with_dsf = bool(rng.random() < 0.5)
        L = 16 if wide else int(rng.choice([16, 8, 4]))
        threads = 512 if wide else 256
        sched = str(rng.choice(["chunks", "sequences"]))
        R = 2 if L == 4 and i % 2 == 0 else 1
        name = (f"s{i:02d}_dk{dk}_dv{dv}_c{chunk}_h{Hk}x{Hv // Hk}_{'bf16' if bf16 else 'f32'}"
                f"_L{L}_t{threads}_r{R}_{sched}")
        cases.append((name, lengths, Hk, Hv, dk, dv, chunk, bf16, with_s0, with_dsf, L,
                      threads, sched, 3000 + i, R))
    return cases


CASES = draw_cases()


def test_sweep_draw_is_fixed_and_admitted():
    """The draw depends on its seed only, and every case is one the library admits."""
    assert draw_cases() == CASES
    for (_, lengths, Hk, Hv, dk, dv, chunk, *_rest) in CASES:
        assert Hv % Hk == 0 and 1 <= dv <= 1024 and Hv * max(dk, dv) <= 1 << 20
        assert dk in (16, 32, 64, 128) and chunk in (16, 32, 64, 128, 256)
        assert all(t >= 0 for t in lengths)


def sweep_workload(case):
    (name, lengths, Hk, Hv, dk, dv, chunk, bf16, with_s0, with_dsf, _L, _t, _s, seed, _R) = case
    w = W.make_packed(name, lengths, Hk=Hk, Hv=Hv, d=dk, chunk=chunk, bf16=bf16, seed=seed)
    if dv != dk:  # v of width d_v from the same recipe
        w.v = W.make_packed(name, lengths, Hk=Hv, Hv=Hv, d=dv, chunk=chunk, bf16=bf16,
                            seed=seed + 1000).v
    s0 = None
    if with_s0:
        g = np.random.default_rng(seed)
        s0 = (0.25 * g.standard_normal((len(lengths), Hv, dv, dk))).astype(np.float32)
    do, dsf = W.cotangents(w, seed + 2000, with_final=with_dsf)
    return w, s0, do, dsf


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sweep_forward_and_backward_match_oracle(case):
    name, L, threads, sched, R = case[0], case[10], case[11], case[12], case[14]
    log(f"sweep: {case}")
    w, s0, do, dsf = sweep_workload(case)
    ro, rcs, rfs = O.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=w.chunk,
                          initial_state=s0, want_chunk_states=True, want_final_state=True)
    ref = O.backward(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, do, chunk=w.chunk,
                     initial_state=s0, dstate_final=dsf)
    d = up_workload(w)
    ds0 = None if s0 is None else up(s0)
    with lanes(L), scan_threads(threads), rows_per_group(R), schedule(sched):
        o, cs = api.trainer_fwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"],
                                chunk=w.chunk, initial_state=ds0,
                                total_chunks=w.total_chunks)
        po, fs = api.prefill(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], chunk=w.chunk,
                             initial_state=ds0)
        got = api.trainer_bwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], up(rcs),
                              up(do), chunk=w.chunk, initial_state=ds0,
                              d_final_state=None if dsf is None else up(dsf),
                              total_chunks=w.total_chunks)
        torch.cuda.synchronize()
    assert_bits(o, ro, f"{name} trainer o")
    assert_bits(cs, rcs, f"{name} trainer chunk states")
    assert_bits(po, ro, f"{name} prefill o")
    assert_bits(fs, rfs, f"{name} prefill final state")
    for g in ("dq", "dk", "dv", "da", "db", "dS0"):
        assert_bits(got[g], ref[g], f"{name} {g}")
