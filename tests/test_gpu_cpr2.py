"""GPU parity of the two-level reading of CPR (gdn_cpr2_* through the C ABI) with the CPU
oracle, bit for bit, and of its three cases with one another.

Small packed batches cover d_k 32, 64 and 128, ragged lengths (empty sequences, lengths
below, at and above multiples of C), GQA, ragged d_v, f32 and bf16 storage, initial states
and every admitted C. Decode runs staggered sequences with idle slots through chunk
boundaries, against the oracle's outputs, chunk states and final states. The trainer
workload (4 x 4096 tokens, 16 heads, d 128, C 64) runs at full size in the launch
configuration that bench.py times, as do the engine-prefill and long-context workloads:
trainer and prefill agree on the device, and the oracle checks sampled (sequence, head)
pairs that it computes alone (for the long context, the first 8192 tokens of two heads). Decode resumes the
engine-decode workload after a 1000-token prefix (mid-chunk, from a boundary state and a
token cache) and must reproduce the trainer's outputs and chunk states step by step, and end
on the prefill's final state.
"""

import zlib

import numpy as np
import pytest
import torch

from bitwise_consistent_linear_amd import api
from bitwise_consistent_linear_amd import workloads as W
from gpu_util import DEV, assert_bits, assert_dev_equal, log, up, up_workload
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def run_trainer(w, d, s0=None):
    return api.cpr2_trainer_fwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"],
                                chunk=w.chunk, initial_state=s0, total_chunks=w.total_chunks)


def run_prefill(w, d, s0=None):
    return api.cpr2_prefill(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], chunk=w.chunk,
                            initial_state=s0, total_chunks=w.total_chunks)


SMALL = [
    # name, lengths, Hk, Hv, d_k, d_v, chunk, bf16, with_s0
    ("d32_ragged_f32", [5, 0, 37, 16, 1, 32], 1, 2, 32, 32, 16, False, True),
    ("d32_gqa2_bf16_c32", [23, 64, 17], 2, 4, 32, 32, 32, True, False),
    ("d64_gqa4_bf16_s0", [100, 3, 48], 1, 4, 64, 64, 16, True, True),
    ("d64_dv40", [33, 50, 64], 1, 2, 64, 40, 16, True, True),
    ("d128_bf16_c64", [130, 64, 0, 77], 2, 2, 128, 128, 64, True, True),
    ("d128_dv72_f32", [45, 19, 96], 2, 4, 128, 72, 32, False, False),
    ("d128_c128", [300, 128, 5], 1, 2, 128, 128, 128, True, True),
    ("d64_c256", [600, 256], 1, 1, 64, 64, 256, False, True),
    ("d32_dv200", [40, 7], 1, 1, 32, 200, 16, True, True),
    ("d128_zero_lengths", [0, 0, 0], 1, 2, 128, 128, 64, True, True),
]


def small_workload(name, lengths, Hk, Hv, dk, dv, chunk, bf16, with_s0):
    seed = zlib.crc32(name.encode()) % 1000
    w = W.make_packed(name, lengths, Hk=Hk, Hv=Hv, d=dk, chunk=chunk, bf16=bf16, seed=600 + seed)
    if dv != dk:  # replace v with a [T, Hv, dv] draw of the same recipe
        w.v = W.make_packed(name, lengths, Hk=Hv, Hv=Hv, d=dv, chunk=chunk, bf16=bf16,
                            seed=1600 + seed).v
    s0 = None
    if with_s0:
        g = np.random.default_rng(seed)
        s0 = (0.25 * g.standard_normal((len(lengths), Hv, dv, dk))).astype(np.float32)
    return w, s0


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases_match_oracle(case):
    w, s0 = small_workload(*case)
    log(f"cpr2 small: {case}")
    ro, rcs, rfs = O.cpr2_scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=w.chunk,
                               initial_state=s0)
    d = up_workload(w)
    ds0 = None if s0 is None else up(s0)
    o, cs = run_trainer(w, d, ds0)
    po, fs = run_prefill(w, d, ds0)
    torch.cuda.synchronize()
    assert_bits(o, ro, f"{case[0]} trainer o")
    assert_bits(cs, rcs, f"{case[0]} trainer chunk states")
    assert_bits(po, ro, f"{case[0]} prefill o")
    assert_bits(fs, rfs, f"{case[0]} prefill final")


def test_two_level_differs_from_one_level():
    """The two readings are distinct contracts: on a multi-chunk sequence their bits differ
    (else the second identity would describe nothing new)."""
    w, s0 = small_workload("differ", [200], 1, 2, 64, 64, 16, True, True)
    d = up_workload(w)
    o2, cs2 = run_trainer(w, d, up(s0))
    o1, cs1 = api.trainer_fwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], chunk=16,
                              initial_state=up(s0))
    torch.cuda.synchronize()
    # the first chunk is computed by the same rows in both readings
    assert torch.equal(o1[:16].view(torch.int32), o2[:16].view(torch.int32))
    assert not torch.equal(cs1.view(torch.int32), cs2.view(torch.int32))


def decode_schedule(lengths, starts):
    """pos [S, N]: sequence n takes token j at step starts[n] + j; -1 elsewhere."""
    S = max(s + l for s, l in zip(starts, lengths))
    pos = np.full((S, len(lengths)), -1, np.int32)
    for n, (s, l) in enumerate(zip(starts, lengths)):
        pos[s:s + l, n] = np.arange(l, dtype=np.int32)
    return pos


@pytest.mark.parametrize("dk,dv,chunk,bf16", [(32, 32, 16, False), (64, 40, 16, True),
                                               (128, 128, 32, True), (128, 72, 64, False)])
def test_decode_staggered_matches_oracle(dk, dv, chunk, bf16):
    lengths, starts = [70, 33, 16, 48], [0, 5, 40, 2]
    if chunk == 64:  # several boundaries per sequence at the larger chunk
        lengths, starts = [200, 130, 64, 5], [0, 17, 3, 60]
    w, s0 = small_workload(f"dec{dk}", lengths, 2, 4, dk, dv, chunk, bf16, True)
    log(f"cpr2 decode: d_k={dk} d_v={dv} C={chunk} bf16={bf16} staggered {lengths}")
    ro, rcs, rfs = O.cpr2_scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=chunk,
                               initial_state=s0)
    pos = decode_schedule(lengths, starts)
    cu = w.cu_seqlens
    coff = np.concatenate([[0], np.cumsum(np.asarray(lengths) // chunk)])
    dt = torch.bfloat16 if bf16 else torch.float32
    dec = api.Cpr2Decoder(len(lengths), 2, 4, dk, dv, chunk, dt, DEV, initial_state=up(s0))
    d = up_workload(w)
    N = len(lengths)
    o_sentinel = torch.full((N, 4, dv), 5.0, device=DEV)
    for s in range(pos.shape[0]):
        tok = np.where(pos[s] >= 0, cu[:-1] + pos[s], 0).astype(np.int64)
        idx = torch.from_numpy(tok).to(DEV)
        rs = torch.full((N, 4, dv, dk), 9.0, device=DEV)
        o = o_sentinel.clone()
        dec.step(up(pos[s]), d["q"][idx].contiguous(), d["k"][idx].contiguous(),
                 d["v"][idx].contiguous(), d["a"][idx].contiguous(), d["b"][idx].contiguous(),
                 o=o, resync_states=rs)
        torch.cuda.synchronize()
        for n in range(N):
            p = int(pos[s, n])
            if p < 0:
                assert bool((o[n] == 5.0).all()), f"idle slot {n} o written at step {s}"
                assert bool((rs[n] == 9.0).all()), f"idle slot {n} resync written at step {s}"
                continue
            assert_bits(o[n], ro[cu[n] + p], f"decode o step {s} seq {n} pos {p}")
            if (p + 1) % chunk == 0:
                assert_bits(rs[n], rcs[coff[n] + (p + 1) // chunk - 1],
                            f"resync step {s} seq {n}")
                assert_bits(dec.boundary[n], rs[n], f"boundary after step {s} seq {n}")
            else:
                assert bool((rs[n] == 9.0).all()), f"resync off-boundary seq {n} step {s}"
    assert_bits(dec.state, rfs, "decode end states vs oracle final states")


def test_final_state_cases():
    """Final state: the boundary state when T_n is a multiple of C (0 included), else the
    rows restarted at the last boundary; T_n < C ends on rows started at the initial
    state."""
    w, s0 = small_workload("finals", [64, 0, 63, 65, 15, 16, 17], 1, 2, 64, 64, 16, True, True)
    _, rcs, rfs = O.cpr2_scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=16, initial_state=s0)
    d = up_workload(w)
    _, fs = run_prefill(w, d, up(s0))
    torch.cuda.synchronize()
    assert_bits(fs, rfs, "final states")
    assert_bits(fs[1], s0[1], "empty sequence keeps its initial state")
    assert_bits(fs[0], rcs[3], "T = 4C ends on S_4")


def test_refused_and_repeat():
    w, s0 = small_workload("rep", [300, 77], 2, 4, 128, 128, 64, True, True)
    d = up_workload(w)
    ds0 = up(s0)
    o = torch.full((w.total_tokens, 4, 128), 3.0, device=DEV)
    with pytest.raises(api.GdnError) as e:
        api.cpr2_trainer_fwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], chunk=64, o=o,
                             identity=api.contract_identity(64, 128))
    assert e.value.status == api.GDN_E_IDENTITY
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())
    first = run_trainer(w, d, ds0)
    for _ in range(3):
        again = run_trainer(w, d, ds0)
        assert_dev_equal(again[0], first[0], "repeat o")
        assert_dev_equal(again[1], first[1], "repeat chunk states")


# ------------------------------------------------------------------- full-size configs

def pair_slice(w, n, h, s0=None):
    """Sequence n, value head h alone (its q/k head is h / (Hv / Hk)): the oracle's input."""
    bos, eos = int(w.cu_seqlens[n]), int(w.cu_seqlens[n + 1])
    hk = h // (w.num_v_heads // w.num_qk_heads)
    sl = slice(bos, eos)
    part = W.Workload(f"{w.name}_n{n}_h{h}", np.array([0, eos - bos], np.int32),
                      np.ascontiguousarray(w.q[sl, hk:hk + 1]),
                      np.ascontiguousarray(w.k[sl, hk:hk + 1]),
                      np.ascontiguousarray(w.v[sl, h:h + 1]),
                      np.ascontiguousarray(w.a[sl, h:h + 1]),
                      np.ascontiguousarray(w.b[sl, h:h + 1]), w.chunk, w.bf16)
    ps0 = None if s0 is None else np.ascontiguousarray(s0[n:n + 1, h:h + 1])
    return part, ps0


def sampled_oracle(w, pairs, o_dev, cs_dev, fs_dev):
    coff = np.concatenate([[0], np.cumsum(w.lengths // w.chunk)])
    for n, h in pairs:
        part, _ = pair_slice(w, n, h)
        ro, rcs, rfs = O.cpr2_scan(part.cu_seqlens, part.q, part.k, part.v, part.a, part.b,
                                   chunk=w.chunk)
        sl = slice(int(w.cu_seqlens[n]), int(w.cu_seqlens[n + 1]))
        assert_bits(o_dev[sl, h], ro[:, 0], f"{w.name} oracle o (n={n}, h={h})")
        assert_bits(cs_dev[coff[n]:coff[n + 1], h], rcs[:, 0],
                    f"{w.name} oracle chunk states (n={n}, h={h})")
        assert_bits(fs_dev[n, h], rfs[0, 0], f"{w.name} oracle final (n={n}, h={h})")


def test_config_trainer_fwd():
    w = W.trainer_fwd()
    log("cpr2 trainer_fwd: N=4 T=4096 H=16 d=128 C=64 bf16")
    d = up_workload(w)
    o, cs = run_trainer(w, d)
    po, fs = run_prefill(w, d)
    torch.cuda.synchronize()
    assert_dev_equal(po, o, "trainer vs prefill o")
    assert_dev_equal(fs, cs.view(4, 64, 16, 128, 128)[:, -1], "prefill final vs last state")
    sampled_oracle(w, [(0, 0), (3, 15), (1, 6)], o, cs, fs)


def test_config_engine_prefill():
    w = W.engine_prefill()
    L = w.lengths
    log(f"cpr2 engine_prefill: N=64 varlen {L.min()}..{L.max()} sum {L.sum()} Hk=16 Hv=32 d=128")
    d = up_workload(w)
    po, fs = run_prefill(w, d)
    o, cs = run_trainer(w, d)
    torch.cuda.synchronize()
    assert_dev_equal(o, po, "trainer vs prefill o")
    # sequences whose length is a multiple of C end on their last chunk state
    coff = np.concatenate([[0], np.cumsum(L // w.chunk)])
    for n in np.flatnonzero(L % w.chunk == 0):
        assert_dev_equal(fs[n], cs[coff[n + 1] - 1], f"final of sequence {n} vs its last state")
    longest, shortest = int(np.argmax(L)), int(np.argmin(L))
    sampled_oracle(w, [(longest, 31), (shortest, 0), (7, 13)], po, cs, fs)


def test_config_long_context():
    w = W.long_context()
    log("cpr2 long_context: T=131072 Hk=16 Hv=32 d=128 C=64")
    d = up_workload(w)
    o, cs = run_trainer(w, d)
    po, fs = run_prefill(w, d)
    torch.cuda.synchronize()
    assert_dev_equal(po, o, "trainer vs prefill o")
    assert_dev_equal(fs, cs[-1:], "prefill final vs last chunk state")
    # the oracle on the first 8192 tokens of two heads: outputs and states there depend on
    # those tokens only
    head = W.Workload("long_head", np.array([0, 8192], np.int32), w.q[:8192], w.k[:8192],
                      w.v[:8192], w.a[:8192], w.b[:8192], 64, True)
    for h in (0, 31):
        part, _ = pair_slice(head, 0, h)
        ro, rcs, _ = O.cpr2_scan(part.cu_seqlens, part.q, part.k, part.v, part.a, part.b,
                                 chunk=64)
        assert_bits(o[:8192, h], ro[:, 0], f"long oracle o (h={h}, first 8192 tokens)")
        assert_bits(cs[:128, h], rcs[:, 0], f"long oracle chunk states (h={h}, first 128)")


def test_config_engine_decode_resumes_mid_chunk():
    w = W.engine_decode()
    prefix, nsteps = w.extra["prefix"], w.extra["steps"]
    C = w.chunk
    log(f"cpr2 engine_decode: N=256 prefix {prefix} (mid-chunk) + {nsteps} decode steps")
    d = up_workload(w)
    o_full, cs_full = run_trainer(w, d)
    _, fs_full = run_prefill(w, d)
    N, T = w.num_seqs, prefix + nsteps
    o_seq = o_full.view(N, T, 32, 128)
    cs_seq = cs_full.view(N, T // C, 32, 128, 128)
    pre, steps = W.split_for_decode(w, prefix)
    dp = up_workload(pre)
    _, pcs = run_trainer(pre, dp)
    _, fs = run_prefill(pre, dp)
    del d, dp
    dec = api.Cpr2Decoder(N, 16, 32, 128, 128, C, torch.bfloat16, DEV)
    nb = prefix // C
    dec.state.copy_(fs)
    dec.boundary.copy_(pcs.view(N, nb, 32, 128, 128)[:, -1])
    tail = prefix - nb * C  # tokens of the chunk in progress go into the cache
    qkv = {key: up(getattr(w, key).reshape(N, T, *getattr(w, key).shape[1:])[:, nb * C:prefix])
           for key in ("k", "v", "a", "b")}
    dec.cache_k[:, :tail].copy_(qkv["k"])
    dec.cache_v[:, :tail].copy_(qkv["v"])
    dec.cache_a[:, :tail].copy_(qkv["a"])
    dec.cache_b[:, :tail].copy_(qkv["b"])
    dst = {k: up(v) for k, v in steps.items()}
    rs = torch.empty_like(fs)
    for s in range(nsteps):
        o = dec.step(dst["pos"][s], dst["q"][s], dst["k"][s], dst["v"][s], dst["a"][s],
                     dst["b"][s], resync_states=rs)
        assert_dev_equal(o, o_seq[:, prefix + s], f"decode step {s} o vs trainer")
        if (prefix + s + 1) % C == 0:
            assert_dev_equal(rs, cs_seq[:, (prefix + s + 1) // C - 1], f"resync step {s}")
    assert_dev_equal(dec.state, fs_full, "decode end state vs prefill of all tokens")
    part, _ = pair_slice(w, 200, 31)
    ro, rcs, _ = O.cpr2_scan(part.cu_seqlens, part.q, part.k, part.v, part.a, part.b, chunk=C)
    assert_bits(o_seq[200, :, 31], ro[:, 0], "oracle o (n=200, h=31)")
    assert_bits(cs_seq[200, :, 31], rcs[:, 0], "oracle chunk states (n=200, h=31)")


def test_decode_steps_in_hip_graph_match_eager():
    """Two-level decode steps (running rows, token cache, listed transitions, boundary
    sweep) captured once into a HIP graph and replayed: every replay, after eager work and
    a sync, gives the bits of the same steps run eagerly (the launches read pos and the
    list from device memory, so one graph serves steps that do and do not end a chunk)."""
    N, Hk, Hv, d, C = 4, 2, 4, 64, 16
    w, s0 = small_workload("graph2", [48] * N, Hk, Hv, d, d, C, True, True)
    _, steps = W.split_for_decode(w, 0)
    dst = {key: up(x) for key, x in steps.items()}
    S = dst["q"].shape[0]

    def make():
        return api.Cpr2Decoder(N, Hk, Hv, d, d, C, torch.bfloat16, DEV, initial_state=up(s0))

    eager = make()
    ref_o, ref_rs = [], []
    for s in range(S):
        rs = torch.zeros((N, Hv, d, d), device=DEV)
        ref_o.append(eager.step(dst["pos"][s], dst["q"][s], dst["k"][s], dst["v"][s],
                                dst["a"][s], dst["b"][s], resync_states=rs).clone())
        ref_rs.append(rs)
    dec = make()
    saved = [t.clone() for t in (dec.state, dec.boundary, dec.cache_k, dec.cache_v,
                                 dec.cache_a, dec.cache_b)]
    outs = [torch.empty((N, Hv, d), device=DEV) for _ in range(S)]
    rss = [torch.zeros((N, Hv, d, d), device=DEV) for _ in range(S)]
    api.cpr2_contract_identity(C, d)  # host work outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(S):
            dec.step(dst["pos"][s], dst["q"][s], dst["k"][s], dst["v"][s], dst["a"][s],
                     dst["b"][s], o=outs[s], resync_states=rss[s])
    for replay in range(3):
        junk = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        for t, src in zip((dec.state, dec.boundary, dec.cache_k, dec.cache_v, dec.cache_a,
                           dec.cache_b), saved):
            t.copy_(src)
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        del junk
        for s in range(S):
            assert_dev_equal(outs[s], ref_o[s], f"replay {replay} step {s} o")
            if (s + 1) % C == 0:
                assert_dev_equal(rss[s], ref_rs[s], f"replay {replay} step {s} resync")
        assert_dev_equal(dec.state, eager.state, f"replay {replay} final state")
        assert_dev_equal(dec.boundary, eager.boundary, f"replay {replay} boundary")


def test_decode_without_resync_buffer():
    """resync_states may be NULL: the steps then give the same outputs, running state and
    boundary state as with a buffer, and write nothing else."""
    N, Hk, Hv, d, C = 3, 1, 2, 32, 16
    w, s0 = small_workload("noresync", [40] * N, Hk, Hv, d, d, C, False, True)
    _, steps = W.split_for_decode(w, 0)
    dst = {key: up(x) for key, x in steps.items()}
    decs = [api.Cpr2Decoder(N, Hk, Hv, d, d, C, torch.float32, DEV, initial_state=up(s0))
            for _ in range(2)]
    for s in range(dst["q"].shape[0]):
        args = (dst["pos"][s], dst["q"][s], dst["k"][s], dst["v"][s], dst["a"][s], dst["b"][s])
        o1 = decs[0].step(*args, resync_states=torch.zeros((N, Hv, d, d), device=DEV))
        o2 = decs[1].step(*args)
        assert_dev_equal(o2, o1, f"step {s} o")
    assert_dev_equal(decs[1].state, decs[0].state, "running state")
    assert_dev_equal(decs[1].boundary, decs[0].boundary, "boundary state")


def test_empty_batch():
    """No sequences at all: every call, one- and two-level, succeeds and launches nothing."""
    cu = torch.zeros(1, dtype=torch.int32, device=DEV)
    q = torch.zeros((0, 1, 64), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device=DEV)
    a = torch.zeros((0, 2), device=DEV)
    outs = [*api.cpr2_trainer_fwd(cu, q, q, v, a, a, chunk=16),
            *api.cpr2_prefill(cu, q, q, v, a, a, chunk=16),
            *api.trainer_fwd(cu, q, q, v, a, a, chunk=16),
            *api.prefill(cu, q, q, v, a, a, chunk=16)]
    pos = torch.zeros(0, dtype=torch.int32, device=DEV)
    outs.append(api.decode_step(pos, q, q, v, a, a, torch.zeros((0, 2, 64, 64), device=DEV),
                                chunk=16))
    dec = api.Cpr2Decoder(0, 1, 2, 64, 64, 16, torch.bfloat16, DEV)
    outs.append(dec.step(pos, q, q, v, a, a))
    torch.cuda.synchronize()
    assert all(t.numel() == 0 for t in outs)
