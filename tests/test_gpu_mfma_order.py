"""How gfx950's binary32 matrix instructions accumulate, established on the GPU.

The linear region and the two-level reading's boundary sweep rest on one property of
v_mfma_f32_16x16x4_f32 and v_mfma_f32_32x32x2_f32: every output is a chain of fused
multiply-adds over k in ascending order, starting from the accumulator, each rounded to
nearest even with subnormals kept. This test runs one wave of each instruction
(libgdn_probe.so, gdn_probe_mfma) on operands with exponents spread over 2^-40..2^40,
products that cancel, subnormal products and signed-zero accumulators, and compares every
output bit for bit with five candidate models computed exactly (exact_fp32, Fraction
arithmetic rounded once per operation): the ascending fma chain must match everywhere, and
each other model - products rounded before adding, one rounding per instruction, a
descending chain inside an instruction, a pairwise sum inside an instruction - must fail
somewhere, so that the inputs tell the models apart."""

import ctypes
import os

import numpy as np
import pytest
import torch

import exact_fp32 as X
from gpu_util import DEV

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "bitwise_consistent_linear_amd", "libgdn_probe.so")


def probe_lib():
    if not os.path.exists(PROBE):
        raise RuntimeError(f"{PROBE} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(PROBE)
    L.gdn_probe_mfma.restype = ctypes.c_int
    L.gdn_probe_mfma.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 4 + [ctypes.c_int,
                                                                         ctypes.c_void_p]
    return L


def operands(n, K, seed):
    g = np.random.default_rng(seed)

    def spread(shape, lo, hi):
        m = g.uniform(1.0, 2.0, shape) * np.where(g.random(shape) < 0.5, -1.0, 1.0)
        return (m * np.exp2(g.integers(lo, hi, shape))).astype(np.float32)

    A = spread((n, K), -20, 21)
    B = spread((K, n), -20, 21)
    C = spread((n, n), -10, 11)
    # products that cancel: the second term of some rows undoes the first
    A[: n // 4, 1] = -A[: n // 4, 0]
    B[1, :] = B[0, :]
    # subnormal products (about 2^-146) onto subnormal accumulators: a block of outputs
    # whose every term lies in the subnormal range
    A[n // 4: n // 2, :] = spread((n // 4, K), -76, -70)
    B[:, n // 2: 3 * n // 4] = spread((K, n // 4), -76, -70)
    C[n // 4: n // 2, n // 2: 3 * n // 4] = spread((n // 4, n // 4), -140, -128)
    # signed zeros: zero operands onto -0.0 and +0.0 accumulators; in row n-1 every
    # product with column 0 is -0.0 (-0.0 times a positive b), so that output stays -0.0
    A[-2:, :] = 0.0
    A[-1, :] = -0.0
    B[:, 0] = np.abs(B[:, 0])
    C[-2:, : n // 2] = -0.0
    C[-2:, n // 2:] = 0.0
    return A, B, C


def models(A, B, C, group):
    """Each candidate's outputs for D = C + A B; group = k per instruction."""
    n, K = A.shape
    out = {name: np.zeros((n, n), np.float32) for name in
           ("fma_chain_ascending", "rounded_products", "one_rounding_per_instruction",
            "fma_chain_descending_in_instruction", "pairwise_in_instruction")}
    for i in range(n):
        for j in range(n):
            a = [float(x) for x in A[i]]
            b = [float(x) for x in B[:, j]]
            c = float(C[i, j])
            acc = c
            for k in range(K):
                acc = X.fma(a[k], b[k], acc)
            out["fma_chain_ascending"][i, j] = acc
            acc = c
            for k in range(K):
                acc = X.add(acc, X.mul(a[k], b[k]))
            out["rounded_products"][i, j] = acc
            acc = c
            for k0 in range(0, K, group):
                exact = X.Fraction(acc) + sum(X.Fraction(a[k]) * X.Fraction(b[k])
                                              for k in range(k0, k0 + group))
                acc = X._round(exact) if exact != 0 else (acc if acc == 0 else 0.0)
            out["one_rounding_per_instruction"][i, j] = acc
            acc = c
            for k0 in range(0, K, group):
                for k in reversed(range(k0, k0 + group)):
                    acc = X.fma(a[k], b[k], acc)
            out["fma_chain_descending_in_instruction"][i, j] = acc
            acc = c
            for k0 in range(0, K, group):
                p = [X.mul(a[k], b[k]) for k in range(k0, k0 + group)]
                while len(p) > 1:
                    p = [X.add(p[t], p[t + 1]) for t in range(0, len(p), 2)]
                acc = X.add(acc, p[0])
            out["pairwise_in_instruction"][i, j] = acc
    return out


@pytest.mark.parametrize("form,n,group", [(0, 16, 4), (1, 32, 2)],
                         ids=["v_mfma_f32_16x16x4_f32", "v_mfma_f32_32x32x2_f32"])
def test_matrix_instructions_are_ascending_fma_chains(form, n, group):
    K = 16
    A, B, C = operands(n, K, 70 + form)
    dA, dB, dC = (torch.from_numpy(x).to(DEV) for x in (A, B, C))
    dD = torch.empty((n, n), dtype=torch.float32, device=DEV)
    L = probe_lib()
    assert L.gdn_probe_mfma(form, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), dD.data_ptr(), K,
                            torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    got = dD.cpu().numpy().view(np.uint32)
    cand = models(A, B, C, group)
    want = cand.pop("fma_chain_ascending").view(np.uint32)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} outputs differ from the ascending fma chain, first {bad[0]}"
    # the inputs separate the models: every other candidate differs from the hardware
    for name, alt in cand.items():
        assert not np.array_equal(alt.view(np.uint32), got), f"{name} is not ruled out"
    # subnormal outputs occur (the subnormal range is exercised, not flushed)
    vals = dD.cpu().numpy()
    assert np.any((vals != 0) & (np.abs(vals) < np.float32(2.0 ** -126)))
    # both signs of zero occur among the outputs
    zeros = vals[vals == 0]
    assert np.any(np.signbit(zeros)) and np.any(~np.signbit(zeros))
