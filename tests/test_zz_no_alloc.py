"""gdn_cpr_trainer_bwd_noalloc (the backward with its workspace in the library's fixed
device array) against gdn_cpr_trainer_bwd (the same kernels with a caller workspace), bit
for bit, through the C ABI: two calls in a row, the second with a smaller input, so the
second reuses the array the first left behind; then the first case again after the array
held the second's contents. Also a call on a side stream, and the same bits as the oracle
for the small case."""

import zlib

import numpy as np
import pytest
import torch

from bitwise_consistent_linear_amd import api
from bitwise_consistent_linear_amd import workloads as W
from gpu_util import DEV, assert_bits, assert_dev_equal, log, up, up_workload
from oracle import oracle as O

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "da", "db", "dS0")


def case(name, lengths, Hk, Hv, d, chunk, bf16):
    seed = zlib.crc32(name.encode()) % 1000
    w = W.make_packed(name, lengths, Hk=Hk, Hv=Hv, d=d, chunk=chunk, bf16=bf16, seed=900 + seed)
    g = np.random.default_rng(seed)
    s0 = (0.25 * g.standard_normal((len(lengths), Hv, d, d))).astype(np.float32)
    do, dsf = W.cotangents(w, 1900 + seed)
    return w, s0, do, dsf


def both(w, s0, do, dsf, stream=None):
    d = up_workload(w)
    ds0 = up(s0)
    _, cs = api.trainer_fwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], chunk=w.chunk,
                            initial_state=ds0)
    kw = dict(chunk=w.chunk, initial_state=ds0, d_final_state=up(dsf),
              total_chunks=w.total_chunks)
    ref = api.trainer_bwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], cs, up(do), **kw)
    got = api.trainer_bwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], cs, up(do),
                          noalloc=True, stream=stream, **kw)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_workspace_call_twice_then_smaller():
    big = case("noalloc_big", [300, 77, 0, 129, 64], 2, 4, 128, 64, True)
    small = case("noalloc_small", [40, 9], 1, 2, 32, 16, False)
    log("noalloc: 5 sequences (570 tokens), Hk=2 Hv=4 d=128 C=64 bf16; then 2 sequences, d=32")
    w, s0, do, dsf = big
    need = api.trainer_bwd_workspace_bytes(
        api.GdnShape(w.num_seqs, 2, 4, 128, 128, 64, api.GDN_DTYPE_BF16), w.total_tokens,
        w.total_chunks)
    assert 0 < need <= api.NOALLOC_MAX_BYTES
    ref, got = both(*big)
    for g in GRADS:
        assert_dev_equal(got[g], ref[g], f"big call {g}")
    ref2, got2 = both(*small)
    for g in GRADS:
        assert_dev_equal(got2[g], ref2[g], f"smaller call {g}")
    # the small case's gradients are also the oracle's
    w2, s02, do2, dsf2 = small
    oref = O.backward(w2.cu_seqlens, w2.q, w2.k, w2.v, w2.a, w2.b, do2, chunk=w2.chunk,
                      initial_state=s02, dstate_final=dsf2)
    for g in GRADS:
        assert_bits(got2[g], oref[g], f"smaller call vs oracle {g}")
    ref3, got3 = both(*big)
    for g in GRADS:
        assert_dev_equal(got3[g], ref[g], f"big call again {g}")
        assert_dev_equal(ref3[g], ref[g], f"workspace call again {g}")


def test_noalloc_on_a_side_stream():
    big = case("noalloc_stream", [200, 150], 1, 2, 64, 64, True)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        ref, got = both(*big, stream=side)
    for g in GRADS:
        assert_dev_equal(got[g], ref[g], f"side stream {g}")


def test_noalloc_refuses_sizes_beyond_the_array_and_leaves_outputs():
    # 2100 tokens of 16 heads at d = 128 need more workspace than the fixed array holds
    w, s0, do, dsf = case("noalloc_refuse", [2100], 16, 16, 128, 64, True)
    need = api.trainer_bwd_workspace_bytes(
        api.GdnShape(1, 16, 16, 128, 128, 64, api.GDN_DTYPE_BF16), w.total_tokens,
        w.total_chunks)
    assert need > api.NOALLOC_MAX_BYTES
    d = up_workload(w)
    _, cs = api.trainer_fwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], chunk=64)
    T = w.total_tokens
    shapes = {"dq": (T, 16, 128), "dk": (T, 16, 128), "dv": (T, 16, 128), "da": (T, 16),
              "db": (T, 16), "dS0": (1, 16, 128, 128)}
    out = {g: torch.full(shp, 7.0, device=DEV) for g, shp in shapes.items()}
    with pytest.raises(api.GdnError) as e:
        api.trainer_bwd(d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], cs, up(do), chunk=64,
                        d_final_state=up(dsf), out=out, noalloc=True)
    assert e.value.status == api.GDN_E_SHAPE
    assert "fixed array" in str(e.value)
    torch.cuda.synchronize()
    assert all(bool((t == 7.0).all()) for t in out.values())
