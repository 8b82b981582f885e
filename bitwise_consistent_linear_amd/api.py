"""ctypes binding of libgdn_cpr.so (the C ABI declared in include/gdn_cpr.h).

Argument marshalling only: the functions check torch tensor dtypes, devices and
contiguity, allocate outputs that the caller did not pass, and call the C entry point of
the same name on the current stream. Every step of the recurrence runs in the library's
HIP kernels; there is no other code path, and a missing library is an error.
"""

from __future__ import annotations

import ctypes
import os
from functools import lru_cache

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdn_cpr.so")

GDN_OK, GDN_E_NULL, GDN_E_SHAPE, GDN_E_UNSUPPORTED, GDN_E_IDENTITY, GDN_E_DEVICE = range(6)
GDN_DTYPE_F32, GDN_DTYPE_BF16 = 0, 1
STATUS_NAMES = {0: "GDN_OK", 1: "GDN_E_NULL", 2: "GDN_E_SHAPE", 3: "GDN_E_UNSUPPORTED",
                4: "GDN_E_IDENTITY", 5: "GDN_E_DEVICE"}


class GdnShape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_qk_heads", ctypes.c_int32),
                ("num_v_heads", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("qkv_dtype", ctypes.c_int32)]


class GdnLinearShape(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("x_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32)]


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.gdn_abi_version.restype = I32
        L.gdn_abi_version.argtypes = []
        L.gdn_contract_string.restype = I32
        L.gdn_contract_string.argtypes = [I32, I32, ctypes.c_char_p, ctypes.c_size_t,
                                          ctypes.POINTER(ctypes.c_size_t)]
        L.gdn_sha256.restype = I32
        L.gdn_sha256.argtypes = [ctypes.c_char_p, ctypes.c_size_t, ctypes.c_char_p]
        L.gdn_contract_identity.restype = I32
        L.gdn_contract_identity.argtypes = [I32, I32, ctypes.c_char_p]
        L.gdn_cpr_trainer_fwd.restype = I32
        L.gdn_cpr_trainer_fwd.argtypes = [ctypes.POINTER(GdnShape), ctypes.c_char_p, P, I64,
                                          P, P, P, P, P, P, P, P, I64, P]
        L.gdn_cpr_prefill.restype = I32
        L.gdn_cpr_prefill.argtypes = [ctypes.POINTER(GdnShape), ctypes.c_char_p, P, I64,
                                      P, P, P, P, P, P, P, P, P]
        L.gdn_cpr_decode_step.restype = I32
        L.gdn_cpr_decode_step.argtypes = [ctypes.POINTER(GdnShape), ctypes.c_char_p, P,
                                          P, P, P, P, P, P, P, P, P]
        L.gdn_cpr_trainer_bwd_workspace.restype = I32
        L.gdn_cpr_trainer_bwd_workspace.argtypes = [ctypes.POINTER(GdnShape), I64, I64,
                                                    ctypes.POINTER(ctypes.c_size_t)]
        L.gdn_cpr_trainer_bwd.restype = I32
        L.gdn_cpr_trainer_bwd.argtypes = [ctypes.POINTER(GdnShape), ctypes.c_char_p, P, I64,
                                          P, P, P, P, P, P, P, I64, P, P,
                                          P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.gdn_cpr_trainer_bwd_noalloc.restype = I32
        L.gdn_cpr_trainer_bwd_noalloc.argtypes = [ctypes.POINTER(GdnShape), ctypes.c_char_p, P,
                                                  I64, P, P, P, P, P, P, P, I64, P, P,
                                                  P, P, P, P, P, P, P]
        L.gdn_linear_fwd.restype = I32
        L.gdn_linear_fwd.argtypes = [ctypes.POINTER(GdnLinearShape), ctypes.c_char_p, P, P, P, P]
        L.gdn_cpr2_contract_string.restype = I32
        L.gdn_cpr2_contract_string.argtypes = [I32, I32, ctypes.c_char_p, ctypes.c_size_t,
                                               ctypes.POINTER(ctypes.c_size_t)]
        L.gdn_cpr2_contract_identity.restype = I32
        L.gdn_cpr2_contract_identity.argtypes = [I32, I32, ctypes.c_char_p]
        L.gdn_cpr2_workspace.restype = I32
        L.gdn_cpr2_workspace.argtypes = [ctypes.POINTER(GdnShape), I64, I64, I32,
                                         ctypes.POINTER(ctypes.c_size_t)]
        L.gdn_cpr2_trainer_fwd.restype = I32
        L.gdn_cpr2_trainer_fwd.argtypes = [ctypes.POINTER(GdnShape), ctypes.c_char_p, P, I64,
                                           P, P, P, P, P, P, P, P, I64, P, ctypes.c_size_t, P]
        L.gdn_cpr2_prefill.restype = I32
        L.gdn_cpr2_prefill.argtypes = [ctypes.POINTER(GdnShape), ctypes.c_char_p, P, I64,
                                       P, P, P, P, P, P, P, P, I64, P, ctypes.c_size_t, P]
        L.gdn_cpr2_decode_step.restype = I32
        L.gdn_cpr2_decode_step.argtypes = [ctypes.POINTER(GdnShape), ctypes.c_char_p, P,
                                           P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                           ctypes.c_size_t, P]
        L.gdn_last_error.restype = ctypes.c_char_p
        L.gdn_last_error.argtypes = []
        _lib = L
    return _lib


def _check(status: int):
    if status != GDN_OK:
        raise GdnError(status, lib().gdn_last_error().decode())


def abi_version() -> int:
    return lib().gdn_abi_version()


def contract_string(chunk: int, d_k: int) -> str:
    n = ctypes.c_size_t(0)
    st = lib().gdn_contract_string(chunk, d_k, None, 0, ctypes.byref(n))
    if st not in (GDN_OK, GDN_E_SHAPE):
        _check(st)
    buf = ctypes.create_string_buffer(n.value + 1)
    _check(lib().gdn_contract_string(chunk, d_k, buf, n.value + 1, ctypes.byref(n)))
    return buf.value.decode()


def sha256(data: bytes) -> bytes:
    out = ctypes.create_string_buffer(32)
    _check(lib().gdn_sha256(data, len(data), out))
    return out.raw


@lru_cache(maxsize=None)
def contract_identity(chunk: int, d_k: int) -> bytes:
    out = ctypes.create_string_buffer(32)
    _check(lib().gdn_contract_identity(chunk, d_k, out))
    return out.raw


# ------------------------------------------------------------------------ tensor helpers

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t, name, dtypes, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")
    return t


def _same_device(*named):
    """Every tensor given (None entries skipped) on the device of the first one: the
    library runs on the current device and cannot check where a pointer lives."""
    present = [(n, t) for n, t in named if t is not None]
    if not present:
        return
    dev = present[0][1].device
    for n, t in present[1:]:
        if t.device != dev:
            raise ValueError(f"{n} is on {t.device}, expected {dev} like {present[0][0]}")


def _qkv(q, k, v):
    torch = _torch()
    dt = (torch.float32, torch.bfloat16)
    _need(q, "q", dt, 3)
    _need(k, "k", dt, 3)
    _need(v, "v", dt, 3)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if q.shape != k.shape:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} differ")
    if v.shape[0] != q.shape[0]:
        raise ValueError(f"v has {v.shape[0]} rows, q and k {q.shape[0]}")
    return GDN_DTYPE_BF16 if q.dtype == torch.bfloat16 else GDN_DTYPE_F32


def _out(t, name, shape):
    """A caller-supplied fp32 output of exactly `shape` (the kernels write all of it)."""
    torch = _torch()
    _need(t, name, (torch.float32,), len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {tuple(t.shape)}")
    return t


def _chunk_states(t, name, total_chunks, Hv, dv, dk):
    torch = _torch()
    _need(t, name, (torch.float32,), 4)
    if t.shape[0] < total_chunks or tuple(t.shape[1:]) != (Hv, dv, dk):
        raise ValueError(f"{name} must be [>= {total_chunks}, {Hv}, {dv}, {dk}], "
                         f"got {tuple(t.shape)}")
    return t


def _shape(N, q, v, chunk, dtype_code):
    return GdnShape(N, q.shape[1], v.shape[1], q.shape[2], v.shape[2], chunk, dtype_code)


def _ab(a, b, T, Hv):
    torch = _torch()
    _need(a, "a", (torch.float32,), 2)
    _need(b, "b", (torch.float32,), 2)
    if tuple(a.shape) != (T, Hv) or tuple(b.shape) != (T, Hv):
        raise ValueError(f"a and b must be [{T}, {Hv}]")


def _state(t, name, N, Hv, dv, dk):
    torch = _torch()
    if t is None:
        return None
    _need(t, name, (torch.float32,), 4)
    if tuple(t.shape) != (N, Hv, dv, dk):
        raise ValueError(f"{name} must be [{N}, {Hv}, {dv}, {dk}], got {tuple(t.shape)}")
    return t


def count_chunks(cu_seqlens, chunk: int) -> int:
    """sum_n floor(T_n / C) from cu_seqlens (reads it back to the host)."""
    c = cu_seqlens.detach().to("cpu").to(_torch().int64)
    return int(((c[1:] - c[:-1]) // chunk).sum())


# ----------------------------------------------------------------------------- entry points

def trainer_fwd(cu_seqlens, q, k, v, a, b, *, chunk, initial_state=None, o=None,
                chunk_states=None, total_chunks=None, identity=None, stream=None):
    """gdn_cpr_trainer_fwd. Returns (o [T, Hv, dv] fp32, chunk_states [total_chunks, Hv, dv, dk])."""
    torch = _torch()
    dt = _qkv(q, k, v)
    _need(cu_seqlens, "cu_seqlens", (torch.int32,), 1)
    N = cu_seqlens.shape[0] - 1
    T, Hv, dv, dk = q.shape[0], v.shape[1], v.shape[2], q.shape[2]
    _ab(a, b, T, Hv)
    _state(initial_state, "initial_state", N, Hv, dv, dk)
    if total_chunks is None:
        total_chunks = count_chunks(cu_seqlens, chunk)
    if o is None:
        o = torch.empty((T, Hv, dv), dtype=torch.float32, device=q.device)
    _out(o, "o", (T, Hv, dv))
    if chunk_states is None:
        chunk_states = torch.empty((total_chunks, Hv, dv, dk), dtype=torch.float32,
                                   device=q.device)
    _chunk_states(chunk_states, "chunk_states", total_chunks, Hv, dv, dk)
    _same_device(("q", q), ("k", k), ("v", v), ("a", a), ("b", b), ("cu_seqlens", cu_seqlens),
                 ("initial_state", initial_state), ("o", o), ("chunk_states", chunk_states))
    shape = _shape(N, q, v, chunk, dt)
    ident = identity if identity is not None else contract_identity(chunk, dk)
    _check(lib().gdn_cpr_trainer_fwd(ctypes.byref(shape), ident, _ptr(cu_seqlens), T,
                                     _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                     _ptr(initial_state), _ptr(o),
                                     _ptr(chunk_states) if total_chunks else None,
                                     total_chunks, _stream(stream)))
    return o, chunk_states


def prefill(cu_seqlens, q, k, v, a, b, *, chunk, initial_state=None, o=None, final_state=None,
            identity=None, stream=None):
    """gdn_cpr_prefill. Returns (o [T, Hv, dv] fp32, final_state [N, Hv, dv, dk])."""
    torch = _torch()
    dt = _qkv(q, k, v)
    _need(cu_seqlens, "cu_seqlens", (torch.int32,), 1)
    N = cu_seqlens.shape[0] - 1
    T, Hv, dv, dk = q.shape[0], v.shape[1], v.shape[2], q.shape[2]
    _ab(a, b, T, Hv)
    _state(initial_state, "initial_state", N, Hv, dv, dk)
    if o is None:
        o = torch.empty((T, Hv, dv), dtype=torch.float32, device=q.device)
    _out(o, "o", (T, Hv, dv))
    if final_state is None:
        final_state = torch.empty((N, Hv, dv, dk), dtype=torch.float32, device=q.device)
    _state(final_state, "final_state", N, Hv, dv, dk)
    _same_device(("q", q), ("k", k), ("v", v), ("a", a), ("b", b), ("cu_seqlens", cu_seqlens),
                 ("initial_state", initial_state), ("o", o), ("final_state", final_state))
    shape = _shape(N, q, v, chunk, dt)
    ident = identity if identity is not None else contract_identity(chunk, dk)
    _check(lib().gdn_cpr_prefill(ctypes.byref(shape), ident, _ptr(cu_seqlens), T, _ptr(q),
                                 _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(initial_state),
                                 _ptr(o), _ptr(final_state), _stream(stream)))
    return o, final_state


def decode_step(pos, q, k, v, a, b, state, *, chunk, o=None, resync_states=None,
                identity=None, stream=None):
    """gdn_cpr_decode_step: one token per sequence; ``state`` is updated in place.

    pos int32 [N]; q, k [N, Hk, dk]; v [N, Hv, dv]; a, b [N, Hv]; state [N, Hv, dv, dk].
    Returns o [N, Hv, dv] fp32.
    """
    torch = _torch()
    dt = _qkv(q, k, v)
    _need(pos, "pos", (torch.int32,), 1)
    N, Hv, dv, dk = q.shape[0], v.shape[1], v.shape[2], q.shape[2]
    if pos.shape[0] != N or v.shape[0] != N:
        raise ValueError("pos, q, k and v must have one row per sequence")
    _ab(a, b, N, Hv)
    if state is None:
        raise ValueError("state is required")
    _state(state, "state", N, Hv, dv, dk)
    _state(resync_states, "resync_states", N, Hv, dv, dk)
    if o is None:
        o = torch.empty((N, Hv, dv), dtype=torch.float32, device=q.device)
    _out(o, "o", (N, Hv, dv))
    _same_device(("q", q), ("k", k), ("v", v), ("a", a), ("b", b), ("pos", pos),
                 ("state", state), ("o", o), ("resync_states", resync_states))
    shape = _shape(N, q, v, chunk, dt)
    ident = identity if identity is not None else contract_identity(chunk, dk)
    _check(lib().gdn_cpr_decode_step(ctypes.byref(shape), ident, _ptr(pos), _ptr(q), _ptr(k),
                                     _ptr(v), _ptr(a), _ptr(b), _ptr(state), _ptr(o),
                                     _ptr(resync_states), _stream(stream)))
    return o


def trainer_bwd_workspace_bytes(shape: GdnShape, total_tokens: int, total_chunks: int) -> int:
    """gdn_cpr_trainer_bwd_workspace: device bytes the backward needs for these sizes."""
    n = ctypes.c_size_t(0)
    _check(lib().gdn_cpr_trainer_bwd_workspace(ctypes.byref(shape), total_tokens,
                                               total_chunks, ctypes.byref(n)))
    return n.value


NOALLOC_MAX_BYTES = 128 << 20  # GDN_CPR_BWD_NOALLOC_MAX_BYTES


def trainer_bwd(cu_seqlens, q, k, v, a, b, chunk_states, d_o, *, chunk, initial_state=None,
                d_final_state=None, total_chunks=None, workspace=None, out=None,
                identity=None, stream=None, noalloc=False):
    """gdn_cpr_trainer_bwd: gradients through trainer_fwd, given d_o [T, Hv, dv] and
    optionally d_final_state [N, Hv, dv, dk].

    chunk_states is trainer_fwd's output for the same inputs. ``workspace`` is a uint8 GPU
    tensor of at least trainer_bwd_workspace_bytes() bytes (allocated here when omitted);
    ``out`` may hold preallocated dq, dk, dv, da, db, dS0 tensors. noalloc=True calls
    gdn_cpr_trainer_bwd_noalloc instead, whose workspace is the library's fixed array
    (sizes up to NOALLOC_MAX_BYTES of workspace); pass every output in ``out`` to make the
    whole call allocation-free.
    Returns a dict with dq, dk [T, Hk, dk]; dv [T, Hv, dv]; da, db [T, Hv];
    dS0 [N, Hv, dv, dk], all fp32.
    """
    torch = _torch()
    dt = _qkv(q, k, v)
    _need(cu_seqlens, "cu_seqlens", (torch.int32,), 1)
    N = cu_seqlens.shape[0] - 1
    T, Hk, Hv, dv, dk = q.shape[0], q.shape[1], v.shape[1], v.shape[2], q.shape[2]
    _ab(a, b, T, Hv)
    _state(initial_state, "initial_state", N, Hv, dv, dk)
    _state(d_final_state, "d_final_state", N, Hv, dv, dk)
    _need(d_o, "d_o", (torch.float32,), 3)
    if tuple(d_o.shape) != (T, Hv, dv):
        raise ValueError(f"d_o must be [{T}, {Hv}, {dv}], got {tuple(d_o.shape)}")
    if total_chunks is None:
        total_chunks = count_chunks(cu_seqlens, chunk)
    _chunk_states(chunk_states, "chunk_states", total_chunks, Hv, dv, dk)
    shapes = {"dq": (T, Hk, dk), "dk": (T, Hk, dk), "dv": (T, Hv, dv), "da": (T, Hv),
              "db": (T, Hv), "dS0": (N, Hv, dv, dk)}
    out = dict(out or {})
    for name, shp in shapes.items():
        if name not in out:
            out[name] = torch.empty(shp, dtype=torch.float32, device=q.device)
        _need(out[name], name, (torch.float32,), len(shp))
        if tuple(out[name].shape) != shp:
            raise ValueError(f"{name} must be {list(shp)}, got {tuple(out[name].shape)}")
    shape = _shape(N, q, v, chunk, dt)
    ident = identity if identity is not None else contract_identity(chunk, dk)
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc=True takes no workspace")
        _same_device(("q", q), ("k", k), ("v", v), ("a", a), ("b", b),
                     ("cu_seqlens", cu_seqlens), ("initial_state", initial_state),
                     ("chunk_states", chunk_states), ("d_o", d_o),
                     ("d_final_state", d_final_state), *[(name, out[name]) for name in shapes])
        _check(lib().gdn_cpr_trainer_bwd_noalloc(
            ctypes.byref(shape), ident, _ptr(cu_seqlens), T, _ptr(q), _ptr(k), _ptr(v),
            _ptr(a), _ptr(b), _ptr(initial_state), _ptr(chunk_states) if total_chunks else None,
            total_chunks, _ptr(d_o), _ptr(d_final_state), _ptr(out["dq"]), _ptr(out["dk"]),
            _ptr(out["dv"]), _ptr(out["da"]), _ptr(out["db"]), _ptr(out["dS0"]),
            _stream(stream)))
        return out
    need = trainer_bwd_workspace_bytes(shape, T, total_chunks)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", (torch.uint8,), 1)
    _same_device(("q", q), ("k", k), ("v", v), ("a", a), ("b", b), ("cu_seqlens", cu_seqlens),
                 ("initial_state", initial_state), ("chunk_states", chunk_states),
                 ("d_o", d_o), ("d_final_state", d_final_state), ("workspace", workspace),
                 *[(name, out[name]) for name in shapes])
    _check(lib().gdn_cpr_trainer_bwd(
        ctypes.byref(shape), ident, _ptr(cu_seqlens), T, _ptr(q), _ptr(k), _ptr(v), _ptr(a),
        _ptr(b), _ptr(initial_state), _ptr(chunk_states) if total_chunks else None,
        total_chunks, _ptr(d_o), _ptr(d_final_state), _ptr(out["dq"]), _ptr(out["dk"]),
        _ptr(out["dv"]), _ptr(out["da"]), _ptr(out["db"]), _ptr(out["dS0"]),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def linear_fwd(x, w, *, y=None, identity=None, stream=None):
    """gdn_linear_fwd: Y = X W of the linear region. x [M, K], w [K, N] (float32 or
    bfloat16, contiguous GPU tensors); returns y float32 [M, N]. The identity defaults to
    the contract identity of (chunk 64, d_k 128); the linear rule is in every one."""
    torch = _torch()
    dt = (torch.float32, torch.bfloat16)
    _need(x, "x", dt, 2)
    _need(w, "w", dt, 2)
    M, K = x.shape
    if w.shape[0] != K:
        raise ValueError(f"x is {tuple(x.shape)} but w is {tuple(w.shape)}")
    N = w.shape[1]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _out(y, "y", (M, N))
    _same_device(("x", x), ("w", w), ("y", y))
    code = {torch.float32: GDN_DTYPE_F32, torch.bfloat16: GDN_DTYPE_BF16}
    shape = GdnLinearShape(M, N, K, code[x.dtype], code[w.dtype])
    ident = identity if identity is not None else contract_identity(64, 128)
    _check(lib().gdn_linear_fwd(ctypes.byref(shape), ident, _ptr(x), _ptr(w), _ptr(y),
                                _stream(stream)))
    return y


# ---------------------------------------------------------------- two-level reading of CPR

def cpr2_contract_string(chunk: int, d_k: int) -> str:
    n = ctypes.c_size_t(0)
    st = lib().gdn_cpr2_contract_string(chunk, d_k, None, 0, ctypes.byref(n))
    if st not in (GDN_OK, GDN_E_SHAPE):
        _check(st)
    buf = ctypes.create_string_buffer(n.value + 1)
    _check(lib().gdn_cpr2_contract_string(chunk, d_k, buf, n.value + 1, ctypes.byref(n)))
    return buf.value.decode()


@lru_cache(maxsize=None)
def cpr2_contract_identity(chunk: int, d_k: int) -> bytes:
    out = ctypes.create_string_buffer(32)
    _check(lib().gdn_cpr2_contract_identity(chunk, d_k, out))
    return out.raw


def cpr2_workspace_bytes(shape: GdnShape, total_tokens: int, total_chunks: int,
                         decode: bool) -> int:
    """gdn_cpr2_workspace: device bytes a two-level call needs for these sizes."""
    n = ctypes.c_size_t(0)
    _check(lib().gdn_cpr2_workspace(ctypes.byref(shape), total_tokens, total_chunks,
                                    1 if decode else 0, ctypes.byref(n)))
    return n.value


def _workspace(workspace, need, device):
    torch = _torch()
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _need(workspace, "workspace", (torch.uint8,), 1)
    return workspace


def _cpr2_batch(prefill_case, cu_seqlens, q, k, v, a, b, chunk, initial_state, o, out_state,
                total_chunks, workspace, identity, stream):
    torch = _torch()
    dt = _qkv(q, k, v)
    _need(cu_seqlens, "cu_seqlens", (torch.int32,), 1)
    N = cu_seqlens.shape[0] - 1
    T, Hv, dv, dk = q.shape[0], v.shape[1], v.shape[2], q.shape[2]
    _ab(a, b, T, Hv)
    _state(initial_state, "initial_state", N, Hv, dv, dk)
    if total_chunks is None:
        total_chunks = count_chunks(cu_seqlens, chunk)
    if o is None:
        o = torch.empty((T, Hv, dv), dtype=torch.float32, device=q.device)
    _out(o, "o", (T, Hv, dv))
    if prefill_case:
        if out_state is None:
            out_state = torch.empty((N, Hv, dv, dk), dtype=torch.float32, device=q.device)
        _state(out_state, "final_state", N, Hv, dv, dk)
    else:
        if out_state is None:
            out_state = torch.empty((total_chunks, Hv, dv, dk), dtype=torch.float32,
                                    device=q.device)
        _chunk_states(out_state, "chunk_states", total_chunks, Hv, dv, dk)
    shape = _shape(N, q, v, chunk, dt)
    workspace = _workspace(workspace, cpr2_workspace_bytes(shape, T, total_chunks, False),
                           q.device)
    _same_device(("q", q), ("k", k), ("v", v), ("a", a), ("b", b), ("cu_seqlens", cu_seqlens),
                 ("initial_state", initial_state), ("o", o), ("state output", out_state),
                 ("workspace", workspace))
    ident = identity if identity is not None else cpr2_contract_identity(chunk, dk)
    fn = lib().gdn_cpr2_prefill if prefill_case else lib().gdn_cpr2_trainer_fwd
    state_ptr = _ptr(out_state) if (prefill_case or total_chunks) else None
    _check(fn(ctypes.byref(shape), ident, _ptr(cu_seqlens), T, _ptr(q), _ptr(k), _ptr(v),
              _ptr(a), _ptr(b), _ptr(initial_state), _ptr(o), state_ptr, total_chunks,
              _ptr(workspace), workspace.numel(), _stream(stream)))
    return o, out_state


def cpr2_trainer_fwd(cu_seqlens, q, k, v, a, b, *, chunk, initial_state=None, o=None,
                     chunk_states=None, total_chunks=None, workspace=None, identity=None,
                     stream=None):
    """gdn_cpr2_trainer_fwd. Returns (o [T, Hv, dv], chunk_states [total_chunks, Hv, dv, dk])."""
    return _cpr2_batch(False, cu_seqlens, q, k, v, a, b, chunk, initial_state, o,
                       chunk_states, total_chunks, workspace, identity, stream)


def cpr2_prefill(cu_seqlens, q, k, v, a, b, *, chunk, initial_state=None, o=None,
                 final_state=None, total_chunks=None, workspace=None, identity=None,
                 stream=None):
    """gdn_cpr2_prefill. Returns (o [T, Hv, dv], final_state [N, Hv, dv, dk])."""
    return _cpr2_batch(True, cu_seqlens, q, k, v, a, b, chunk, initial_state, o,
                       final_state, total_chunks, workspace, identity, stream)


class Cpr2Decoder:
    """The per-sequence buffers of gdn_cpr2_decode_step for N slots: running state,
    boundary state, the C-token cache and the workspace, all on one GPU. ``step`` applies
    one token to every slot whose pos is >= 0 and returns o [N, Hv, dv]."""

    def __init__(self, N, Hk, Hv, dk, dv, chunk, dtype, device, initial_state=None):
        torch = _torch()
        self.N, self.Hk, self.Hv, self.dk, self.dv, self.chunk = N, Hk, Hv, dk, dv, chunk
        self.dtype = dtype
        f32 = dict(dtype=torch.float32, device=device)
        self.state = torch.zeros((N, Hv, dv, dk), **f32)
        if initial_state is not None:
            self.state.copy_(initial_state)
        self.boundary = self.state.clone()
        self.cache_k = torch.zeros((N, chunk, Hk, dk), dtype=dtype, device=device)
        self.cache_v = torch.zeros((N, chunk, Hv, dv), dtype=dtype, device=device)
        self.cache_a = torch.zeros((N, chunk, Hv), **f32)
        self.cache_b = torch.zeros((N, chunk, Hv), **f32)
        code = GDN_DTYPE_BF16 if dtype == torch.bfloat16 else GDN_DTYPE_F32
        self.shape = GdnShape(N, Hk, Hv, dk, dv, chunk, code)
        self.workspace = _workspace(None, cpr2_workspace_bytes(self.shape, 0, 0, True), device)

    def step(self, pos, q, k, v, a, b, *, o=None, resync_states=None, identity=None,
             stream=None):
        torch = _torch()
        _qkv(q, k, v)
        _need(pos, "pos", (torch.int32,), 1)
        if (pos.shape[0], q.shape[0], v.shape[0]) != (self.N,) * 3 or q.dtype != self.dtype:
            raise ValueError("pos, q, k and v must have one row per slot, in the decoder's dtype")
        if tuple(q.shape[1:]) != (self.Hk, self.dk) or tuple(v.shape[1:]) != (self.Hv, self.dv):
            raise ValueError("q, k or v does not match the decoder's heads and widths")
        _ab(a, b, self.N, self.Hv)
        _state(resync_states, "resync_states", self.N, self.Hv, self.dv, self.dk)
        if o is None:
            o = torch.empty((self.N, self.Hv, self.dv), dtype=torch.float32, device=q.device)
        _out(o, "o", (self.N, self.Hv, self.dv))
        _same_device(("the decoder's state", self.state), ("q", q), ("k", k), ("v", v),
                     ("a", a), ("b", b), ("pos", pos), ("o", o),
                     ("resync_states", resync_states))
        ident = identity if identity is not None else cpr2_contract_identity(self.chunk,
                                                                             self.dk)
        _check(lib().gdn_cpr2_decode_step(
            ctypes.byref(self.shape), ident, _ptr(pos), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
            _ptr(b), _ptr(self.state), _ptr(self.boundary), _ptr(self.cache_k),
            _ptr(self.cache_v), _ptr(self.cache_a), _ptr(self.cache_b), _ptr(o),
            _ptr(resync_states), _ptr(self.workspace), self.workspace.numel(),
            _stream(stream)))
        return o
