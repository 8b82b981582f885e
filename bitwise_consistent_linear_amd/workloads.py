"""Seeded synthetic inputs for the GDN-CPR workloads (shared by tests, bench and smoke).

This module holds no arithmetic of the recurrence: it only draws inputs. Both the HIP path
and the CPU oracle consume the same stored bytes, so the generator's own rounding (the
L2 normalisation of k, the cast to bfloat16) never shows up as a difference between them.

Recipe: numpy PCG64 streams from ``SeedSequence(seed).spawn(6)``, one per drawn quantity in
the order lengths, q, k, v, a, b; each tensor is drawn in fixed blocks of whole rows (2**22
elements when the row length divides it), block j from the j-th child of its stream, so the values do not depend on thread count.
  q, k ~ N(0, 1) per element, k scaled to unit L2 norm per (token, q/k head) in float32;
  v ~ N(0, 1); a ~ U(a_lo, 1); b ~ U(0, 1); initial state zero unless a test says otherwise.
  bfloat16 storage is float32 rounded to nearest even, kept as uint16 bit patterns.
Varlen lengths: lognormal(ln(mean) - 1/2, 1) draws, scaled by bisection so that the
floored, clipped lengths sum to at most the token budget, the remainder then handed out one
token at a time round-robin to sequences still below the upper clip.

The IsoExec pages measure only end to end on an RL workload (a 35B hybrid model on a maths
dataset); they give no Gated DeltaNet shapes. These configurations stand in for it.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even) and return the 16-bit patterns (no NaNs here)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << np.uint32(16)).view(np.float32)


def lognormal_lengths(rng: np.random.Generator, n: int, total: int, lo: int, hi: int,
                      mean: float) -> np.ndarray:
    raw = rng.lognormal(np.log(mean) - 0.5, 1.0, n)

    def sized(scale):
        return np.clip(np.floor(raw * scale), lo, hi).astype(np.int64)

    if n * lo > total or n * hi < total:
        raise ValueError("token budget cannot be met within the clip range")
    s_lo, s_hi = 0.0, 1.0
    while sized(s_hi).sum() < total:
        s_hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (s_lo + s_hi)
        if sized(mid).sum() <= total:
            s_lo = mid
        else:
            s_hi = mid
    lengths = sized(s_lo)
    i = 0
    while lengths.sum() < total:
        if lengths[i % n] < hi:
            lengths[i % n] += 1
        i += 1
    return lengths


@dataclass
class Workload:
    """A packed batch: q, k [T, Hk, d]; v [T, Hv, d]; a, b [T, Hv]; cu_seqlens [N+1]."""

    name: str
    cu_seqlens: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    a: np.ndarray
    b: np.ndarray
    chunk: int
    bf16: bool
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return self.cu_seqlens.size - 1

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens.astype(np.int64))

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def num_qk_heads(self) -> int:
        return self.k.shape[1]

    @property
    def num_v_heads(self) -> int:
        return self.v.shape[1]

    @property
    def d_k(self) -> int:
        return self.k.shape[2]

    @property
    def d_v(self) -> int:
        return self.v.shape[2]

    @property
    def total_chunks(self) -> int:
        return int((self.lengths // self.chunk).sum())


_BLOCK = 1 << 22


def _threads() -> int:
    try:
        import os
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except Exception:  # pragma: no cover
        return 4


def _draw(seq: np.random.SeedSequence, shape, kind: str, bf16: bool = False,
          unit_rows: bool = False, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    """Fill an array of ``shape`` block by block from children of ``seq``.

    kind "normal": N(0,1) float32, optionally scaled to unit L2 norm along the last axis and
    stored as bf16 bits; kind "uniform": U(lo, hi) float32.
    """
    from concurrent.futures import ThreadPoolExecutor

    size = int(np.prod(shape))
    row = shape[-1]
    blk = _BLOCK - _BLOCK % row  # whole rows per block
    out = np.empty(shape, np.uint16 if bf16 else np.float32)
    flat = out.reshape(-1)
    nblk = (size + blk - 1) // blk
    kids = seq.spawn(nblk)

    def fill(j):
        g = np.random.Generator(np.random.PCG64(kids[j]))
        m = min(blk, size - j * blk)
        if kind == "normal":
            x = g.standard_normal(m, dtype=np.float32)
            if unit_rows:
                r = x.reshape(-1, row)
                r /= np.sqrt(np.sum(r * r, axis=1, dtype=np.float32), dtype=np.float32)[:, None]
        else:
            x = g.uniform(lo, hi, m).astype(np.float32)
        flat[j * blk:j * blk + m] = f32_to_bf16_bits(x) if bf16 else x

    if nblk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def _streams(seed: int):
    return np.random.SeedSequence(seed).spawn(6)


def make_packed(name: str, lengths, Hk: int, Hv: int, d: int, chunk: int, bf16: bool,
                seed: int, a_lo: float = 0.9) -> Workload:
    """Draw q, k, v, a, b for the given sequence lengths from the streams of ``seed``."""
    st = _streams(seed)
    lengths = np.asarray(lengths, np.int64)
    cu = np.zeros(lengths.size + 1, np.int64)
    np.cumsum(lengths, out=cu[1:])
    if cu[-1] >= 2**31:
        raise ValueError("total tokens must fit in int32")
    T = int(cu[-1])
    q = _draw(st[1], (T, Hk, d), "normal", bf16)
    k = _draw(st[2], (T, Hk, d), "normal", bf16, unit_rows=True)
    v = _draw(st[3], (T, Hv, d), "normal", bf16)
    a = _draw(st[4], (T, Hv), "uniform", lo=a_lo, hi=1.0)
    b = _draw(st[5], (T, Hv), "uniform", lo=0.0, hi=1.0)
    return Workload(name, cu.astype(np.int32), q, k, v, a, b, chunk, bf16)


def cotangents(w: Workload, seed: int, with_final: bool = True, final_scale: float = 0.1):
    """Seeded upstream gradients for the backward: dL/do ~ N(0, 1) float32 [T, Hv, d_v]
    and, if ``with_final``, dL/dS_final ~ final_scale * N(0, 1) float32 [N, Hv, d_v, d_k]
    (else None), from the two children of ``SeedSequence(seed)``, drawn as above."""
    st = np.random.SeedSequence(seed).spawn(2)
    do = _draw(st[0], (w.total_tokens, w.num_v_heads, w.d_v), "normal")
    dsf = None
    if with_final:
        dsf = _draw(st[1], (w.num_seqs, w.num_v_heads, w.d_v, w.d_k), "normal")
        dsf *= np.float32(final_scale)
    return do, dsf


def make_linear(M: int, N: int, K: int, bf16: bool, seed: int):
    """Inputs of the linear region: x [M, K] ~ N(0, 1) and w [K, N] ~ N(0, 1/K) (the usual
    scale of a layer's weights), from the first two children of SeedSequence(seed), drawn
    as above (bf16 as uint16 bit patterns). Row m of x is drawn from the same stream
    positions whatever M is, so a smaller M gives a prefix of the same rows."""
    st = np.random.SeedSequence(seed).spawn(2)
    x = _draw(st[0], (M, K), "normal", bf16)
    w32 = _draw(st[1], (K, N), "normal")
    w32 *= np.float32(1.0 / np.sqrt(K))
    w = f32_to_bf16_bits(w32) if bf16 else w32
    return x, w


# ----------------------------------------------------------------------------------------
# The five workload configurations.

def tiny() -> Workload:
    """N=1, T=64, 2 heads, d_k=d_v=16, C=16, all float32 (seed 0)."""
    return make_packed("tiny", [64], Hk=2, Hv=2, d=16, chunk=16, bf16=False, seed=0)


def trainer_fwd() -> Workload:
    """4 equal sequences of 4096 tokens, 16 heads, d=128, C=64, bf16 q/k/v (seed 1)."""
    return make_packed("trainer_fwd", [4096] * 4, Hk=16, Hv=16, d=128, chunk=64, bf16=True,
                       seed=1)


def engine_prefill(total: int = 262144, n: int = 64) -> Workload:
    """64 lognormal-length sequences in [256, 16384] summing to 262144 tokens; 16 q/k heads
    shared by 32 v heads, d=128, C=64, bf16 (seed 2)."""
    rng = np.random.Generator(np.random.PCG64(_streams(2)[0]))
    lengths = lognormal_lengths(rng, n, total, 256, 16384, mean=total / n)
    return make_packed("engine_prefill", lengths, Hk=16, Hv=32, d=128, chunk=64, bf16=True,
                       seed=2)


def engine_decode(n: int = 256, prefix: int = 1000, steps: int = 512) -> Workload:
    """256 sequences of prefix + steps tokens (drawn up front), 32 v / 16 q/k heads, d=128,
    C=64, bf16 (seed 3). The first ``prefix`` tokens go through prefill, the rest through
    decode steps."""
    w = make_packed("engine_decode", [prefix + steps] * n, Hk=16, Hv=32, d=128, chunk=64,
                    bf16=True, seed=3)
    w.extra.update(prefix=prefix, steps=steps)
    return w


def long_context(T: int = 131072, prefix: int = 65536, steps: int = 256) -> Workload:
    """One sequence of 131072 tokens, 32 v / 16 q/k heads, d=128, C=64, bf16, a ~ U(0.95, 1)
    (seed 4). Decode runs ``steps`` tokens after a ``prefix``-token prefill."""
    w = make_packed("long_context", [T], Hk=16, Hv=32, d=128, chunk=64, bf16=True, seed=4,
                    a_lo=0.95)
    w.extra.update(prefix=prefix, steps=steps)
    return w


CONFIGS = {
    "tiny": tiny,
    "trainer_fwd": trainer_fwd,
    "engine_prefill": engine_prefill,
    "engine_decode": engine_decode,
    "long_context": long_context,
}


def split_for_decode(w: Workload, prefix: int):
    """Equal-length packed batch -> (prefix Workload, per-step arrays).

    Per-step arrays have a leading step axis: q, k [S, N, Hk, d]; v [S, N, Hv, d];
    a, b [S, N, Hv]; pos [S, N] (tokens absorbed before the step).
    """
    L = w.lengths
    if not np.all(L == L[0]) or prefix > L[0]:
        raise ValueError("split_for_decode needs equal lengths of at least the prefix")
    N, T = w.num_seqs, int(L[0])

    def per_seq(x):
        return x.reshape(N, T, *x.shape[1:])

    def head(x):
        return np.ascontiguousarray(per_seq(x)[:, :prefix]).reshape(N * prefix, *x.shape[1:])

    def tail(x):
        return np.ascontiguousarray(np.swapaxes(per_seq(x)[:, prefix:], 0, 1))

    cu = (np.arange(N + 1, dtype=np.int64) * prefix).astype(np.int32)
    pre = Workload(w.name + "_prefix", cu, head(w.q), head(w.k), head(w.v), head(w.a),
                   head(w.b), w.chunk, w.bf16)
    steps = {"q": tail(w.q), "k": tail(w.k), "v": tail(w.v), "a": tail(w.a), "b": tail(w.b)}
    steps["pos"] = np.repeat((prefix + np.arange(T - prefix, dtype=np.int32))[:, None], N, axis=1)
    return pre, steps
