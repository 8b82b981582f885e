"""GPU parity of the linear region (gdn_linear_fwd through the C ABI) with the CPU oracle,
bit for bit, and its batch invariance.

Small products cover ragged m and n (tiles that end part-way in both directions), n that
does and does not allow vector loads of W, every dtype mix, k from 512 to 4096 (leaves of
1 to 8 stages), both stage depths (64-k stages for bf16 inputs with k a multiple of 1024
and n of 128, 32-k stages otherwise), signed zeros and denormals. The bench-size product (16384 x 4096 x 4096,
bf16) is compared with the oracle on sampled rows, and rows must not change with m.
"""

import numpy as np
import pytest
import torch

from bitwise_consistent_linear_amd import api
from bitwise_consistent_linear_amd import workloads as W
from gpu_util import DEV, assert_bits, assert_dev_equal, log, up
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def run(x, w):
    y = api.linear_fwd(up(x), up(w))
    torch.cuda.synchronize()
    return y


SMALL = [
    # M, N, K, x bf16, w bf16, seed
    (1, 1, 512, True, True, 1),
    (5, 33, 512, False, False, 2),
    (64, 128, 1024, True, True, 3),
    (130, 200, 1536, True, False, 4),
    (65, 129, 512, False, True, 5),
    (3, 8, 4096, True, True, 6),
    (200, 64, 2048, False, False, 7),
    # bf16 inputs with K a multiple of 1024 and N of 128 take 64-k stages: ragged M, several
    # column tiles; the neighbours that do not (K = 1536, N = 200) take 32-k stages
    (70, 256, 2048, True, True, 8),
    (129, 384, 1024, True, True, 9),
    (40, 128, 1536, True, True, 10),
    (17, 200, 1024, True, True, 11),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in SMALL])
def test_linear_small_matches_oracle(case):
    M, N, K, xb, wb, seed = case
    log(f"linear small: M={M} N={N} K={K} x_bf16={xb} w_bf16={wb}")
    x, w = W.make_linear(M, N, K, xb, seed)
    if xb != wb:  # the other dtype for w, same values rounded or widened
        _, w = W.make_linear(M, N, K, wb, seed)
    assert_bits(run(x, w), O.linear(x, w), f"linear {case}")


def test_linear_signed_zeros_and_denormals():
    g = np.random.default_rng(11)
    M, N, K = 33, 40, 512
    # products near 2^-140 and sums of a few hundred of them stay below 2^-126: the leaf
    # chains, the tree and the outputs all work in the denormal range
    x = (g.standard_normal((M, K)) * 2.0 ** g.integers(-45, -40, (M, K))).astype(np.float32)
    w = (g.standard_normal((K, N)) * 2.0 ** g.integers(-100, -95, (K, N))).astype(np.float32)
    x[g.random((M, K)) < 0.2] = -0.0
    x[g.random((M, K)) < 0.1] = 0.0
    w[:, 3] = -0.0  # a column of negative zeros: the output's sign of zero is fixed too
    x[5] = -0.0
    log("linear: signed zeros and denormal products")
    y = run(x, w)
    want = O.linear(x, w)
    assert_bits(y, want, "zeros/denormals")
    assert np.any((want != 0) & (np.abs(want) < np.float32(2.0 ** -126))), "no denormal output"


def test_linear_batch_invariance():
    N, K = 96, 1024
    x, w = W.make_linear(1000, N, K, True, 21)
    log("linear: batch invariance over M in {1, 7, 64, 65, 1000}")
    dw = up(w)
    full = api.linear_fwd(up(x), dw)
    for M in (1, 7, 64, 65):
        part = api.linear_fwd(up(x[:M]), dw)
        assert_dev_equal(part, full[:M], f"M={M} rows vs M=1000")
    torch.cuda.synchronize()
    assert_bits(full, O.linear(x, w), "M=1000 vs oracle")


def test_linear_batch_invariance_64k_stages():
    """The same at a shape that takes 64-k stages (bf16, K = 2048, N = 256); the oracle
    checks that its bits are the 32-k stage kernel's too."""
    N, K = 256, 2048
    x, w = W.make_linear(300, N, K, True, 22)
    log("linear: batch invariance over M in {1, 129, 300} with 64-k stages")
    dw = up(w)
    full = api.linear_fwd(up(x), dw)
    for M in (1, 129):
        part = api.linear_fwd(up(x[:M]), dw)
        assert_dev_equal(part, full[:M], f"M={M} rows vs M=300")
    torch.cuda.synchronize()
    assert_bits(full, O.linear(x, w), "M=300 vs oracle")


def test_linear_bench_size_sampled_rows():
    M, N, K = 16384, 4096, 4096
    log("linear: 16384 x 4096 x 4096 bf16, sampled rows vs oracle, repeat determinism")
    x, w = W.make_linear(M, N, K, True, 31)
    dx, dw = up(x), up(w)
    y = api.linear_fwd(dx, dw)
    y2 = api.linear_fwd(dx, dw)
    torch.cuda.synchronize()
    assert_dev_equal(y2, y, "repeat")
    rows = np.array([0, 1, 63, 64, 8191, 16320, 16383] +
                    list(np.random.default_rng(5).integers(0, M, 9)))
    want = O.linear(x[rows], w)
    assert_bits(y[torch.from_numpy(rows).to(DEV)], want, "sampled rows")
    # the same rows alone (m = 16): batch invariance at full size
    alone = api.linear_fwd(up(np.ascontiguousarray(x[rows])), dw)
    assert_dev_equal(alone, y[torch.from_numpy(rows).to(DEV)], "rows alone vs in the batch")


def test_linear_refused_leaves_output():
    x, w = W.make_linear(4, 8, 512, True, 41)
    y = torch.full((4, 8), 3.0, device=DEV)
    with pytest.raises(api.GdnError) as e:
        api.linear_fwd(up(x[:, :500].copy()), up(w[:500].copy()), y=y)
    assert e.value.status == api.GDN_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
