"""Helpers for the GPU parity tests: uploads, bitwise comparisons, runs of the three cases."""

import os

import numpy as np
import torch

from bitwise_consistent_linear_amd import api

DEV = torch.device("cuda:0")
LANES = (16, 8, 4)


def log(msg):
    print(f"[gpu-test] {msg}", flush=True)


def up(x):
    """numpy array -> device tensor; uint16 arrays are bfloat16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x).to(DEV)


def up_workload(w):
    return {"cu": up(w.cu_seqlens), "q": up(w.q), "k": up(w.k), "v": up(w.v), "a": up(w.a),
            "b": up(w.b)}


def host_bits(x):
    if torch.is_tensor(x):
        x = x.detach().to("cpu").numpy()
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def assert_bits(got, want, label):
    g, w = host_bits(got), host_bits(want)
    assert g.shape == w.shape, f"{label}: shape {g.shape} vs {w.shape}"
    if not np.array_equal(g, w):
        bad = np.argwhere(g != w)
        idx = tuple(bad[0])
        gf = g.view(np.float32)[idx]
        wf = w.view(np.float32)[idx]
        raise AssertionError(f"{label}: {len(bad)} of {g.size} differ; first at {idx}: "
                             f"{gf!r} (0x{g[idx]:08x}) vs {wf!r} (0x{w[idx]:08x})")


def assert_dev_equal(x, y, label):
    """Bitwise equality of two device float32 tensors, compared on the device."""
    assert x.shape == y.shape, f"{label}: shape {tuple(x.shape)} vs {tuple(y.shape)}"
    xi, yi = x.view(torch.int32), y.view(torch.int32)
    if not torch.equal(xi, yi):
        n = int((xi != yi).sum())
        first = tuple(int(t) for t in torch.nonzero(xi != yi)[0])
        raise AssertionError(f"{label}: {n} of {x.numel()} differ; first at {first}")


class lanes:
    """Context manager: run the library with a given number of lanes per state row."""

    def __init__(self, L):
        self.L = L

    def __enter__(self):
        self.old = os.environ.get("GDN_CPR_LANES_PER_ROW")
        os.environ["GDN_CPR_LANES_PER_ROW"] = str(self.L)

    def __exit__(self, *exc):
        if self.old is None:
            os.environ.pop("GDN_CPR_LANES_PER_ROW", None)
        else:
            os.environ["GDN_CPR_LANES_PER_ROW"] = self.old


class schedule:
    """Context manager: run the backward's chunk pass with a given schedule, "chunks" (one
    workgroup per chunk, after the state pass) or "sequences" (one per sequence, sweeping
    its chunks in reverse)."""

    def __init__(self, name):
        self.name = name

    def __enter__(self):
        self.old = os.environ.get("GDN_CPR_BWD_SCHEDULE")
        os.environ["GDN_CPR_BWD_SCHEDULE"] = self.name

    def __exit__(self, *exc):
        if self.old is None:
            os.environ.pop("GDN_CPR_BWD_SCHEDULE", None)
        else:
            os.environ["GDN_CPR_BWD_SCHEDULE"] = self.old


SCHEDULES = ("chunks", "sequences")


class scan_threads:
    """Context manager: with "256", keep 256-thread scan workgroups where the library would
    take 512 (two waves per SIMD at 16 lanes per row)."""

    def __init__(self, n):
        self.n = str(n)

    def __enter__(self):
        self.old = os.environ.get("GDN_CPR_SCAN_THREADS")
        os.environ["GDN_CPR_SCAN_THREADS"] = self.n

    def __exit__(self, *exc):
        if self.old is None:
            os.environ.pop("GDN_CPR_SCAN_THREADS", None)
        else:
            os.environ["GDN_CPR_SCAN_THREADS"] = self.old


class rows_per_group:
    """Context manager: at 4 lanes per row in 256-thread scan workgroups, hold R rows (1 or
    2) in each group of lanes; without it the library picks."""

    def __init__(self, R):
        self.R = str(R)

    def __enter__(self):
        self.old = os.environ.get("GDN_CPR_ROWS_PER_GROUP")
        os.environ["GDN_CPR_ROWS_PER_GROUP"] = self.R

    def __exit__(self, *exc):
        if self.old is None:
            os.environ.pop("GDN_CPR_ROWS_PER_GROUP", None)
        else:
            os.environ["GDN_CPR_ROWS_PER_GROUP"] = self.old


def decode_steps(dev_steps, state, chunk, s_range=None, resync=True):
    """Run decode steps; yields (step index, o, resync tensor or None)."""
    S = dev_steps["q"].shape[0]
    rs = torch.empty_like(state) if resync else None
    for s in range(S) if s_range is None else s_range:
        o = api.decode_step(dev_steps["pos"][s], dev_steps["q"][s], dev_steps["k"][s],
                            dev_steps["v"][s], dev_steps["a"][s], dev_steps["b"][s], state,
                            chunk=chunk, resync_states=rs)
        yield s, o, rs


def up_steps(steps):
    return {k: up(v) for k, v in steps.items()}
