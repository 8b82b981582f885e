"""GPU parity of the backward (gdn_cpr_trainer_bwd through the C ABI) with the CPU oracle,
bit for bit.

Small cases cover ragged and empty sequences, lengths that are and are not multiples of C
and of the 8-token recompute sub-block, GQA, every d_k, f32 and bf16 storage, ragged d_v
(row blocks that end part-way, d_v below 16, up to 1024 rows), initial states, dL/dS_final
present or absent, every admitted C (chunks of 128 and 256 are processed as 64-token
segments, so lengths end part-way through a segment and in every segment), every
lanes-per-row value of the state pass, and both
schedules of the chunk pass (one workgroup per chunk after the state pass, or one per
sequence sweeping its chunks in reverse). The
trainer-size configuration (4 x 4096 tokens, 16 heads, d = 128, C = 64) is compared with
the oracle over every output. The chunk states fed to the backward are the oracle's, so
these tests do not lean on the forward kernels.
"""

import zlib

import numpy as np
import pytest
import torch

from bitwise_consistent_linear_amd import api
from bitwise_consistent_linear_amd import workloads as W
from gpu_util import (DEV, LANES, SCHEDULES, assert_bits, assert_dev_equal, lanes, log, schedule,
                      up, up_workload)
from oracle import oracle as O

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "da", "db", "dS0")


def oracle_bwd(w, s0, do, dsf):
    ref = O.backward(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, do, chunk=w.chunk,
                     initial_state=s0, dstate_final=dsf)
    _, cs, _ = O.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=w.chunk, initial_state=s0,
                      want_chunk_states=True, want_final_state=True)
    return ref, cs


def run_bwd(w, d, cs, do, dsf, s0=None, workspace=None):
    return api.trainer_bwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], cs, do,
                           chunk=w.chunk, initial_state=s0, d_final_state=dsf,
                           total_chunks=w.total_chunks, workspace=workspace)


def assert_grads(got, ref, label):
    for g in GRADS:
        assert_bits(got[g], ref[g], f"{label} {g}")


def case_workload(name, lengths, Hk, Hv, dk, dv, chunk, bf16, with_s0, with_dsf):
    seed = zlib.crc32(name.encode()) % 1000
    w = W.make_packed(name, lengths, Hk=Hk, Hv=Hv, d=dk, chunk=chunk, bf16=bf16, seed=600 + seed)
    if dv != dk:  # v of width d_v from the same recipe
        w.v = W.make_packed(name, lengths, Hk=Hv, Hv=Hv, d=dv, chunk=chunk, bf16=bf16,
                            seed=1600 + seed).v
    s0 = None
    if with_s0:
        g = np.random.default_rng(seed)
        s0 = (0.25 * g.standard_normal((len(lengths), Hv, dv, dk))).astype(np.float32)
    do, dsf = W.cotangents(w, 2600 + seed, with_final=with_dsf)
    return w, s0, do, dsf


SMALL = [
    # name, lengths, Hk, Hv, d_k, d_v, chunk, bf16, with_s0, with_dsf
    ("tiny_d16_c16_f32", [64], 2, 2, 16, 16, 16, False, False, False),
    ("d16_ragged_c16", [5, 0, 37, 16, 1], 1, 2, 16, 16, 16, False, True, True),
    ("d32_gqa2_bf16_c32", [23, 64, 17, 96], 2, 4, 32, 32, 32, True, False, True),
    ("d64_gqa4_c16_s0", [100, 3, 48], 1, 4, 64, 64, 16, True, True, True),
    ("d128_bf16_c64", [130, 64, 0, 77, 200], 2, 2, 128, 128, 64, True, True, True),
    ("d128_f32_c64_tails", [71, 135, 8, 9], 1, 2, 128, 128, 64, False, True, False),
    ("d64_dv40_c16", [33, 50], 1, 2, 64, 40, 16, True, True, True),
    ("d128_dv72_gqa2_c32", [45, 19], 2, 4, 128, 72, 32, False, False, True),
    ("d32_dv7_c16", [50, 9], 1, 1, 32, 7, 16, False, True, True),
    ("d16_dv300_c16", [40], 1, 1, 16, 300, 16, True, True, True),
    ("d16_dv1024_c64", [70], 1, 1, 16, 1024, 64, False, False, True),
    ("d128_empty_batch_c64", [0, 0, 0], 1, 2, 128, 128, 64, True, True, True),
    ("d32_c128_segments", [300, 128, 65, 0, 129], 1, 2, 32, 32, 128, True, True, True),
    ("d128_c128_f32", [200, 57], 1, 1, 128, 128, 128, False, False, True),
    ("d64_dv40_c256", [520, 255, 64, 193], 2, 2, 64, 40, 256, True, True, True),
    ("d128_bf16_c256_gqa", [256, 300], 1, 2, 128, 128, 256, True, True, False),
    ("d16_dv300_c256", [270], 1, 1, 16, 300, 256, False, True, True),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_bwd_small_cases_match_oracle(case):
    w, s0, do, dsf = case_workload(*case)
    log(f"bwd small: {case}")
    ref, cs = oracle_bwd(w, s0, do, dsf)
    d = up_workload(w)
    dcs, ddo = up(cs), up(do)
    ddsf = None if dsf is None else up(dsf)
    ds0 = None if s0 is None else up(s0)
    for L in LANES:
        with lanes(L), schedule("chunks"):
            got = run_bwd(w, d, dcs, ddo, ddsf, ds0)
            torch.cuda.synchronize()
        assert_grads(got, ref, f"{case[0]} L={L} chunks")
    with schedule("sequences"):
        got = run_bwd(w, d, dcs, ddo, ddsf, ds0)
        torch.cuda.synchronize()
    assert_grads(got, ref, f"{case[0]} sequences")


def test_bwd_many_sequences_plan_carry_and_unranked_state_pass():
    """1100 sequences: the plan's prefix sums carry over several 256-wide passes, and the
    state pass takes sequences in natural order (more than 1024 to rank)."""
    g = np.random.default_rng(77)
    lengths = g.integers(0, 40, 1100)
    w, s0, do, dsf = case_workload("many_seqs", list(lengths), 1, 2, 16, 16, 16, True, True, True)
    log(f"bwd many sequences: N=1100 T={w.total_tokens}")
    ref, cs = oracle_bwd(w, s0, do, dsf)
    d = up_workload(w)
    for sched in SCHEDULES:
        with schedule(sched):
            got = run_bwd(w, d, up(cs), up(do), up(dsf), up(s0))
            torch.cuda.synchronize()
        assert_grads(got, ref, f"many sequences, {sched}")


def test_bwd_workspace_contents_do_not_matter():
    """A workspace full of NaN bit patterns, reused across calls of different sizes, gives
    the same bits as a fresh one."""
    case = ("ws_reuse", [90, 31, 64], 1, 2, 64, 40, 32, True, True, True)
    w, s0, do, dsf = case_workload(*case)
    log("bwd workspace reuse")
    ref, cs = oracle_bwd(w, s0, do, dsf)
    d = up_workload(w)
    sh = api.GdnShape(w.num_seqs, 1, 2, 64, 40, 32, api.GDN_DTYPE_BF16)
    need = api.trainer_bwd_workspace_bytes(sh, w.total_tokens, w.total_chunks)
    ws = torch.full((need + 4096,), 0xFF, dtype=torch.uint8, device=DEV)
    for sched in SCHEDULES + SCHEDULES:
        with schedule(sched):
            got = run_bwd(w, d, up(cs), up(do), up(dsf), up(s0), workspace=ws)
            torch.cuda.synchronize()
        assert_grads(got, ref, f"reused workspace, {sched}")
    w2, s02, do2, dsf2 = case_workload("ws_reuse_small", [17], 1, 2, 64, 40, 32, True, True, True)
    ref2, cs2 = oracle_bwd(w2, s02, do2, dsf2)
    got2 = run_bwd(w2, up_workload(w2), up(cs2), up(do2), up(dsf2), up(s02), workspace=ws)
    torch.cuda.synchronize()
    assert_grads(got2, ref2, "reused workspace, smaller call")


def test_bwd_refuses_unadmitted_chunk_and_leaves_outputs():
    w, s0, do, dsf = case_workload("refuse", [130], 1, 1, 32, 32, 64, False, False, True)
    d = up_workload(w)
    o, cs = api.trainer_fwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], chunk=64)
    out = {g: None for g in GRADS}
    sentinel = torch.full((130, 1, 32), 7.0, device=DEV)
    with pytest.raises(api.GdnError) as e:
        api.trainer_bwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], cs, up(do),
                        chunk=100, total_chunks=1, d_final_state=up(dsf),
                        out={"dq": sentinel})
    assert e.value.status == api.GDN_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())
    del out


# ------------------------------------------------------------------- trainer-size config

@pytest.fixture(scope="module")
def trainer_case():
    w = W.trainer_fwd()
    do, dsf = W.cotangents(w, 11)
    log("bwd trainer config: N=4 T=4096 H=16 d=128 C=64 bf16; oracle over every output")
    ref = O.backward(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, do, chunk=w.chunk,
                     dstate_final=dsf)
    return w, do, dsf, ref


def test_bwd_config_trainer_matches_oracle(trainer_case):
    """Automatic choices (the sequence schedule here: 4 x 16 x 4 row blocks fill the
    CUs), then the chunk schedule at every lanes-per-row value, all against the oracle or
    the first result."""
    w, do, dsf, ref = trainer_case
    d = up_workload(w)
    o, cs = api.trainer_fwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], chunk=w.chunk)
    ddo, ddsf = up(do), up(dsf)
    got = run_bwd(w, d, cs, ddo, ddsf)
    torch.cuda.synchronize()
    assert_grads(got, ref, "trainer config")
    again = run_bwd(w, d, cs, ddo, ddsf)
    for L in LANES:
        with lanes(L), schedule("chunks"):
            other = run_bwd(w, d, cs, ddo, ddsf)
        for g in GRADS:
            assert_dev_equal(other[g], got[g], f"chunks L={L} vs automatic {g}")
    with schedule("sequences"):
        other = run_bwd(w, d, cs, ddo, ddsf)
    for g in GRADS:
        assert_dev_equal(other[g], got[g], f"sequences vs automatic {g}")
        assert_dev_equal(again[g], got[g], f"repeat {g}")


@pytest.mark.parametrize("chunk", [16, 32, 128, 256])
def test_bwd_config_trainer_other_chunks_same_bits(trainer_case, chunk):
    """C only selects which states the forward stores: the gradients keep their bits."""
    w, do, dsf, ref = trainer_case
    log(f"bwd trainer config at C={chunk}")
    d = up_workload(w)
    w.chunk, saved = chunk, w.chunk
    try:
        o, cs = api.trainer_fwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], chunk=chunk)
        got = run_bwd(w, d, cs, up(do), up(dsf))
        torch.cuda.synchronize()
    finally:
        w.chunk = saved
    assert_grads(got, ref, f"trainer config C={chunk}")
