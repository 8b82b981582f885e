"""The Python binding's own refusals (the C ABI cannot see tensor sizes): a caller-supplied
output of the wrong size, a short v, chunk states of the wrong row shape, or a tensor on
another device raise ValueError before anything is launched, so nothing outside the
tensors is read or written; every output passed in keeps its contents."""

import pytest
import torch

from bitwise_consistent_linear_amd import api
from bitwise_consistent_linear_amd import workloads as W
from gpu_util import DEV, up, up_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def small():
    w = W.make_packed("binding", [40, 24], Hk=1, Hv=2, d=32, chunk=16, bf16=False, seed=3)
    return w, up_workload(w)


def _args(d):
    return d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"]


def test_trainer_refuses_wrong_o_and_chunk_states(small):
    w, d = small
    T = w.total_tokens
    short_o = torch.full((T - 1, 2, 32), 5.0, device=DEV)
    with pytest.raises(ValueError, match="o must be"):
        api.trainer_fwd(*_args(d), chunk=16, o=short_o)
    assert bool((short_o == 5.0).all())
    cs = torch.full((w.total_chunks, 2, 32, 16), 5.0, device=DEV)  # rows of d_k 16, not 32
    with pytest.raises(ValueError, match="chunk_states must be"):
        api.trainer_fwd(*_args(d), chunk=16, chunk_states=cs)
    assert bool((cs == 5.0).all())
    few = torch.full((w.total_chunks - 1, 2, 32, 32), 5.0, device=DEV)
    with pytest.raises(ValueError, match="chunk_states must be"):
        api.trainer_fwd(*_args(d), chunk=16, chunk_states=few)


def test_scan_refuses_short_v(small):
    w, d = small
    cu, q, k, v, a, b = _args(d)
    with pytest.raises(ValueError, match="v has"):
        api.prefill(cu, q, k, v[:-1].contiguous(), a, b, chunk=16)
    with pytest.raises(ValueError, match="v has"):
        api.trainer_fwd(cu, q, k, v[:-3].contiguous(), a, b, chunk=16)


def test_prefill_refuses_wrong_o_and_host_tensor(small):
    w, d = small
    o = torch.full((w.total_tokens, 2, 31), 5.0, device=DEV)
    with pytest.raises(ValueError, match="o must be"):
        api.prefill(*_args(d), chunk=16, o=o)
    assert bool((o == 5.0).all())
    cu, q, k, v, a, b = _args(d)
    with pytest.raises(ValueError, match="GPU"):
        api.prefill(cu, q, k, v, a.cpu(), b, chunk=16)


def test_decode_refuses_wrong_o(small):
    w, d = small
    N, Hv, dv, dk = 2, 2, 32, 32
    state = torch.zeros((N, Hv, dv, dk), device=DEV)
    pos = torch.zeros(N, dtype=torch.int32, device=DEV)
    q, k, v = d["q"][:N].contiguous(), d["k"][:N].contiguous(), d["v"][:N].contiguous()
    a, b = d["a"][:N].contiguous(), d["b"][:N].contiguous()
    o = torch.full((N, Hv, dv - 1), 5.0, device=DEV)
    with pytest.raises(ValueError, match="o must be"):
        api.decode_step(pos, q, k, v, a, b, state, chunk=16, o=o)
    assert bool((o == 5.0).all()) and bool((state == 0).all())
    with pytest.raises(ValueError, match="state is required"):
        api.decode_step(pos, q, k, v, a, b, None, chunk=16)


def test_two_level_and_linear_refuse_wrong_outputs(small):
    w, d = small
    o = torch.full((w.total_tokens + 1, 2, 32), 5.0, device=DEV)
    with pytest.raises(ValueError, match="o must be"):
        api.cpr2_trainer_fwd(*_args(d), chunk=16, o=o)
    cs = torch.full((w.total_chunks, 2, 16, 32), 5.0, device=DEV)
    with pytest.raises(ValueError, match="chunk_states must be"):
        api.cpr2_trainer_fwd(*_args(d), chunk=16, chunk_states=cs)
    assert bool((o == 5.0).all()) and bool((cs == 5.0).all())
    x, wm = W.make_linear(8, 16, 512, True, 5)
    y = torch.full((8, 15), 5.0, device=DEV)
    with pytest.raises(ValueError, match="y must be"):
        api.linear_fwd(up(x), up(wm), y=y)
    assert bool((y == 5.0).all())
