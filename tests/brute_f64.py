"""Dense float64 form of the gated delta rule, used to pin the oracle's semantics.

Whole matrices, no row decomposition, no reduction tree:
    S_t = a_t * S_{t-1} @ (I - b_t k_t k_t^T) + b_t v_t k_t^T,    o_t = S_t @ q_t
with S of shape [d_v, d_k] per (sequence, value head), q/k head h // (Hv // Hk).
This is the gated delta rule as published (Yang, Kautz & Hatamizadeh, "Gated Delta
Networks", ICLR 2025), which the IsoExec pages name as the model the CPR kernels compute.
"""

import numpy as np


def as_f64(x):
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def scan_f64(cu_seqlens, q, k, v, a, b, chunk, initial_state=None):
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    a, b = a.astype(np.float64), b.astype(np.float64)
    N = len(cu_seqlens) - 1
    T, Hk, dk = k.shape
    Hv, dv = v.shape[1:]
    G = Hv // Hk
    o = np.zeros((T, Hv, dv))
    finals = np.zeros((N, Hv, dv, dk))
    chunks = []
    eye = np.eye(dk)
    for n in range(N):
        bos, eos = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
        S = np.zeros((Hv, dv, dk)) if initial_state is None else initial_state[n].astype(np.float64)
        for t in range(bos, eos):
            for h in range(Hv):
                kk = k[t, h // G]
                S[h] = a[t, h] * S[h] @ (eye - b[t, h] * np.outer(kk, kk)) + b[t, h] * np.outer(v[t, h], kk)
                o[t, h] = S[h] @ q[t, h // G]
            if (t - bos + 1) % chunk == 0:
                chunks.append(S.copy())
        finals[n] = S
    cs = np.stack(chunks) if chunks else np.zeros((0, Hv, dv, dk))
    return o, cs, finals


def loss_f64(cu_seqlens, q, k, v, a, b, s0, do, dsf):
    """L = sum(do * o) + sum(dsf * S_final), everything in float64 (dense form)."""
    o, _, fs = scan_f64(cu_seqlens, q, k, v, a, b, 1 << 30, s0)
    return float(np.sum(o * do.astype(np.float64)) + np.sum(fs * dsf.astype(np.float64)))


def grads_torch_f64(cu_seqlens, q, k, v, a, b, s0, do, dsf):
    """Exact gradients of loss_f64 by torch autograd in float64 on the CPU (dense form)."""
    import torch

    def t(x):
        return torch.tensor(as_f64(x), dtype=torch.float64, requires_grad=True)

    tq, tk, tv, ta, tb, ts0 = t(q), t(k), t(v), t(a), t(b), t(s0)
    N = len(cu_seqlens) - 1
    Hk, dk = k.shape[1], k.shape[2]
    Hv = v.shape[1]
    G = Hv // Hk
    eye = torch.eye(dk, dtype=torch.float64)
    tdo = torch.tensor(do, dtype=torch.float64)
    loss = torch.zeros((), dtype=torch.float64)
    for n in range(N):
        S = ts0[n]
        for t_ in range(int(cu_seqlens[n]), int(cu_seqlens[n + 1])):
            heads = []
            for h in range(Hv):
                kk = tk[t_, h // G]
                Sh = ta[t_, h] * S[h] @ (eye - tb[t_, h] * torch.outer(kk, kk)) \
                    + tb[t_, h] * torch.outer(tv[t_, h], kk)
                loss = loss + (tdo[t_, h] * (Sh @ tq[t_, h // G])).sum()
                heads.append(Sh)
            S = torch.stack(heads)
        loss = loss + (torch.tensor(dsf[n], dtype=torch.float64) * S).sum()
    loss.backward()
    return {"dq": tq.grad.numpy(), "dk": tk.grad.numpy(), "dv": tv.grad.numpy(),
            "da": ta.grad.numpy(), "db": tb.grad.numpy(), "dS0": ts0.grad.numpy()}
