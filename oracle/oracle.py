"""CPU oracle for CPR Gated DeltaNet (gated delta rule in the contract's binary32 order).

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may use this module; the product path never does.

The arithmetic lives in ``gdn_oracle.c`` (plain C, ``-ffp-contract=off``, ``fmaf`` where
the contract fuses). This module only builds it with gcc and marshals numpy arrays. It
imports nothing from the HIP package and the HIP package imports nothing from here.

Sources: the recurrence is the gated delta rule (Yang, Kautz & Hatamizadeh, "Gated Delta
Networks", ICLR 2025); IsoExec's pages (agentlenshq.com, section "Chunkwise-Parallel
Recurrent (CPR) Gated DeltaNet") fix the three cases and the C-token resync, and the same
page's section on parallel invariance fixes a fixed binary reduction tree with fp32
accumulation. The readings taken where the pages are silent are listed at the top of
``gdn_oracle.c``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile an oracle source with gcc into a shared library and return its path."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, src, "-lm"], check=True)
        os.replace(tmp, out)
    return out


class Oracle:
    """ctypes view of one build of gdn_oracle.c (the default build, or a test's mutant)."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_scan.argtypes = [I] * 7 + [P] * 10 + [I]
        lib.oracle_scan.restype = I
        lib.oracle_scan_pairs.argtypes = [I] * 7 + [P] * 7 + [I, P, P, P, P, P, I]
        lib.oracle_scan_pairs.restype = I
        lib.oracle_decode_step.argtypes = [I] * 7 + [P] * 9
        lib.oracle_decode_step.restype = I
        lib.oracle_backward.argtypes = [I] * 7 + [P] * 15 + [I]
        lib.oracle_backward.restype = I
        lib.oracle_cpr2_scan.argtypes = [I] * 7 + [P] * 10 + [I]
        lib.oracle_cpr2_scan.restype = I
        lib.oracle_cpr2_decode_step.argtypes = [I] * 7 + [P] * 14
        lib.oracle_cpr2_decode_step.restype = I
        lib.oracle_linear.argtypes = [I, I, I, I, I, P, P, P, I]
        lib.oracle_linear.restype = I
        lib.oracle_dot.argtypes = [P, P, I]
        lib.oracle_dot.restype = ctypes.c_float
        self.lib = lib
        self.path = lib_path

    def dot(self, x: np.ndarray, y: np.ndarray) -> np.float32:
        """The contract dot product of two binary32 vectors (length a multiple of 16)."""
        x = _c(x, np.float32)
        y = _c(y, np.float32)
        assert x.shape == y.shape and x.ndim == 1 and x.size % 16 == 0
        return np.float32(self.lib.oracle_dot(_ptr(x), _ptr(y), x.size))

    def scan(self, cu_seqlens, q, k, v, a, b, *, chunk, initial_state=None, want_o=True,
             want_chunk_states=False, want_final_state=False, nthreads=None):
        """Recurrence over a packed batch; returns (o, chunk_states, final_state), None if unasked.

        cu_seqlens int32 [N+1]; q, k [T, Hk, dk]; v [T, Hv, dv] (float32, or uint16 holding
        bf16); a, b float32 [T, Hv]; initial_state float32 [N, Hv, dv, dk] or None (zeros).
        """
        cu = _c(cu_seqlens, np.int32)
        q, k, v = _c(q), _c(k), _c(v)
        a, b = _c(a, np.float32), _c(b, np.float32)
        dt = _dtype_code(q)
        assert _dtype_code(k) == dt and _dtype_code(v) == dt
        N = cu.size - 1
        T, Hk, dk = k.shape
        Hv, dv = v.shape[1], v.shape[2]
        lengths = np.diff(cu.astype(np.int64))
        total_chunks = int((lengths // chunk).sum())
        s0 = _c(initial_state, np.float32)
        o = np.empty((T, Hv, dv), np.float32) if want_o else None
        cs = np.empty((total_chunks, Hv, dv, dk), np.float32) if want_chunk_states else None
        fs = np.empty((N, Hv, dv, dk), np.float32) if want_final_state else None
        rc = self.lib.oracle_scan(N, Hk, Hv, dk, dv, chunk, dt, _ptr(cu), _ptr(q), _ptr(k),
                                  _ptr(v), _ptr(a), _ptr(b), _ptr(s0), _ptr(o), _ptr(cs),
                                  _ptr(fs), nthreads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_scan rejected its arguments (rc={rc})")
        return o, cs, fs

    def scan_pairs(self, cu_seqlens, q, k, v, a, b, pairs, *, chunk, initial_state=None,
                   nthreads=None):
        """Recurrence for selected (n, h) pairs only.

        Returns one dict per pair: {"o": [T_n, dv], "chunk_states": [floor(T_n/C), dv, dk],
        "final_state": [dv, dk]}.
        """
        cu = _c(cu_seqlens, np.int32)
        q, k, v = _c(q), _c(k), _c(v)
        a, b = _c(a, np.float32), _c(b, np.float32)
        dt = _dtype_code(q)
        N = cu.size - 1
        T, Hk, dk = k.shape
        Hv, dv = v.shape[1], v.shape[2]
        pairs = np.asarray(pairs, np.int32).reshape(-1, 2)
        pn = np.ascontiguousarray(pairs[:, 0])
        ph = np.ascontiguousarray(pairs[:, 1])
        lengths = np.diff(cu.astype(np.int64))
        sel_len = lengths[pn]
        o = np.empty((int(sel_len.sum()), dv), np.float32)
        cs = np.empty((int((sel_len // chunk).sum()), dv, dk), np.float32)
        fs = np.empty((len(pn), dv, dk), np.float32)
        s0 = _c(initial_state, np.float32)
        rc = self.lib.oracle_scan_pairs(N, Hk, Hv, dk, dv, chunk, dt, _ptr(cu), _ptr(q),
                                        _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(s0), len(pn),
                                        _ptr(pn), _ptr(ph), _ptr(o), _ptr(cs), _ptr(fs),
                                        nthreads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_scan_pairs rejected its arguments (rc={rc})")
        out, o_at, c_at = [], 0, 0
        for p, L in enumerate(sel_len):
            nc = int(L // chunk)
            out.append({"o": o[o_at:o_at + L], "chunk_states": cs[c_at:c_at + nc],
                        "final_state": fs[p]})
            o_at += int(L)
            c_at += nc
        return out

    def backward(self, cu_seqlens, q, k, v, a, b, do, *, chunk, initial_state=None,
                 dstate_final=None, nthreads=None):
        """Gradients given dL/do [T, Hv, dv] and dL/dS_final [N, Hv, dv, dk] (None = 0).

        Returns dict with dq, dk [T, Hk, dk]; dv [T, Hv, dv]; da, db [T, Hv];
        dS0 [N, Hv, dv, dk] (all float32), in the backward contract's fixed order.
        """
        cu = _c(cu_seqlens, np.int32)
        q, k, v = _c(q), _c(k), _c(v)
        a, b = _c(a, np.float32), _c(b, np.float32)
        do = _c(do, np.float32)
        dt = _dtype_code(q)
        N = cu.size - 1
        T, Hk, dk = k.shape
        Hv, dv = v.shape[1], v.shape[2]
        s0 = _c(initial_state, np.float32)
        dsf = _c(dstate_final, np.float32)
        out = {"dq": np.zeros((T, Hk, dk), np.float32), "dk": np.zeros((T, Hk, dk), np.float32),
               "dv": np.zeros((T, Hv, dv), np.float32), "da": np.zeros((T, Hv), np.float32),
               "db": np.zeros((T, Hv), np.float32),
               "dS0": np.zeros((N, Hv, dv, dk), np.float32)}
        rc = self.lib.oracle_backward(N, Hk, Hv, dk, dv, chunk, dt, _ptr(cu), _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(a), _ptr(b), _ptr(s0), _ptr(do), _ptr(dsf),
                                      _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                      _ptr(out["da"]), _ptr(out["db"]), _ptr(out["dS0"]),
                                      nthreads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_backward rejected its arguments (rc={rc})")
        return out

    def cpr2_scan(self, cu_seqlens, q, k, v, a, b, *, chunk, initial_state=None,
                  nthreads=None):
        """Two-level CPR over a packed batch. Returns (o [T, Hv, dv], chunk_states
        [sum floor(T_n/C), Hv, dv, dk], final_state [N, Hv, dv, dk]), all float32."""
        cu = _c(cu_seqlens, np.int32)
        q, k, v = _c(q), _c(k), _c(v)
        a, b = _c(a, np.float32), _c(b, np.float32)
        dt = _dtype_code(q)
        N = cu.size - 1
        T, Hk, dk = k.shape
        Hv, dv = v.shape[1], v.shape[2]
        s0 = _c(initial_state, np.float32)
        total_chunks = int(((cu[1:].astype(np.int64) - cu[:-1]) // chunk).sum())
        o = np.zeros((T, Hv, dv), np.float32)
        cs = np.zeros((total_chunks, Hv, dv, dk), np.float32)
        fs = np.zeros((N, Hv, dv, dk), np.float32)
        rc = self.lib.oracle_cpr2_scan(N, Hk, Hv, dk, dv, chunk, dt, _ptr(cu), _ptr(q), _ptr(k),
                                       _ptr(v), _ptr(a), _ptr(b), _ptr(s0), _ptr(o), _ptr(cs),
                                       _ptr(fs), nthreads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_cpr2_scan rejected its arguments (rc={rc})")
        return o, cs, fs

    def cpr2_decoder(self, N, Hk, Hv, dk, dv, *, chunk, initial_state=None):
        """State of a two-level decode: running rows, boundary state and the token cache."""
        st = np.zeros((N, Hv, dv, dk), np.float32) if initial_state is None else \
            np.array(initial_state, np.float32, copy=True)
        return {"state": st, "boundary": st.copy(),
                "ck": np.zeros((N, chunk, Hk, dk), np.float32),
                "cv": np.zeros((N, chunk, Hv, dv), np.float32),
                "ca": np.zeros((N, chunk, Hv), np.float32),
                "cb": np.zeros((N, chunk, Hv), np.float32), "chunk": chunk}

    def cpr2_decode_step(self, dec, pos, q, k, v, a, b):
        """One two-level decode step; updates ``dec`` in place; returns (o, resync)."""
        pos = _c(pos, np.int32)
        q, k, v = _c(q), _c(k), _c(v)
        a, b = _c(a, np.float32), _c(b, np.float32)
        N, Hk, dk = k.shape
        Hv, dv = v.shape[1], v.shape[2]
        o = np.zeros((N, Hv, dv), np.float32)
        rs = np.zeros((N, Hv, dv, dk), np.float32)
        rc = self.lib.oracle_cpr2_decode_step(
            N, Hk, Hv, dk, dv, dec["chunk"], _dtype_code(q), _ptr(pos), _ptr(q), _ptr(k),
            _ptr(v), _ptr(a), _ptr(b), _ptr(dec["state"]), _ptr(dec["boundary"]),
            _ptr(dec["ck"]), _ptr(dec["cv"]), _ptr(dec["ca"]), _ptr(dec["cb"]), _ptr(o), _ptr(rs))
        if rc != 0:
            raise ValueError(f"oracle_cpr2_decode_step rejected its arguments (rc={rc})")
        return o, rs

    def linear(self, x, w, *, nthreads=None):
        """Y = X W of the linear region: X [M, K], W [K, N] (float32, or bfloat16 as uint16
        bit patterns); every Y[m, n] is the contract dot of row m of X and column n of W.
        Returns Y float32 [M, N]."""
        x, w = _c(x), _c(w)
        M, K = x.shape
        K2, N = w.shape
        if K2 != K:
            raise ValueError(f"x is [{M}, {K}] but w is [{K2}, {N}]")
        y = np.zeros((M, N), np.float32)
        rc = self.lib.oracle_linear(M, N, K, _dtype_code(x), _dtype_code(w), _ptr(x), _ptr(w),
                                    _ptr(y), nthreads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_linear rejected its arguments (rc={rc})")
        return y

    def decode_step(self, pos, q, k, v, a, b, state, *, chunk, want_resync=True):
        """One decode step; updates ``state`` in place and returns (o, resync or None).

        pos int32 [N] (tokens already absorbed; negative = idle slot); q, k [N, Hk, dk];
        v [N, Hv, dv]; a, b [N, Hv]; state float32 [N, Hv, dv, dk], C-contiguous.
        """
        pos = _c(pos, np.int32)
        q, k, v = _c(q), _c(k), _c(v)
        a, b = _c(a, np.float32), _c(b, np.float32)
        assert state.dtype == np.float32 and state.flags.c_contiguous
        dt = _dtype_code(q)
        N, Hk, dk = k.shape
        Hv, dv = v.shape[1], v.shape[2]
        o = np.zeros((N, Hv, dv), np.float32)
        rs = np.zeros_like(state) if want_resync else None
        rc = self.lib.oracle_decode_step(N, Hk, Hv, dk, dv, chunk, dt, _ptr(pos), _ptr(q),
                                         _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(state),
                                         _ptr(o), _ptr(rs))
        if rc != 0:
            raise ValueError(f"oracle_decode_step rejected its arguments (rc={rc})")
        return o, rs


def _ptr(x):
    return None if x is None else x.ctypes.data


def _dtype_code(arr) -> int:
    if arr.dtype == np.float32:
        return 0
    if arr.dtype == np.uint16:  # bfloat16 bit patterns
        return 1
    raise TypeError(f"q/k/v must be float32 or uint16 (bf16 bits), got {arr.dtype}")


def _c(x, dtype=None):
    if x is None:
        return None
    x = np.asarray(x)
    return np.ascontiguousarray(x if dtype is None else x.astype(dtype, copy=False))


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


_default = None


def get() -> Oracle:
    """The oracle built from the committed source (built on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build()
        _default = Oracle(_LIB)
    return _default


def dot(x, y):
    return get().dot(x, y)


def scan(*args, **kw):
    return get().scan(*args, **kw)


def scan_pairs(*args, **kw):
    return get().scan_pairs(*args, **kw)


def decode_step(*args, **kw):
    return get().decode_step(*args, **kw)


def backward(*args, **kw):
    return get().backward(*args, **kw)


def linear(*args, **kw):
    return get().linear(*args, **kw)


def cpr2_scan(*args, **kw):
    return get().cpr2_scan(*args, **kw)
