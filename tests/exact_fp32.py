"""Exact-rational binary32 emulator of the contract's operation order (tiny inputs only).

Every value is a binary32 number held exactly in a Python float. Every operation is done
exactly with ``fractions.Fraction`` and then rounded once to binary32 with round to nearest,
ties to even, including the subnormal range; the sign of an exact zero follows IEEE 754.
It shares nothing with the C oracle or the HIP kernels: it pins that they really perform
the stated sequence of correctly rounded operations (no hidden contraction, a fused fma,
the stated tree).
"""

from fractions import Fraction
import math

_EMIN = -126
_PREC = 24


def _round(r: Fraction) -> float:
    if r == 0:
        return 0.0
    neg = r < 0
    a = -r if neg else r
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, _EMIN) - (_PREC - 1))
    scaled = a / quantum
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = float(n * quantum)
    if val >= 2.0 ** 128:
        val = math.inf
    return -val if neg else val


def _neg0(x: float) -> bool:
    return math.copysign(1.0, x) < 0


def mul(x: float, y: float) -> float:
    if x == 0 or y == 0:
        return -0.0 if _neg0(x) != _neg0(y) else 0.0
    return _round(Fraction(x) * Fraction(y))


def add(x: float, y: float) -> float:
    r = Fraction(x) + Fraction(y)
    if r == 0:
        return -0.0 if (x == 0 and y == 0 and _neg0(x) and _neg0(y)) else 0.0
    return _round(r)


def sub(x: float, y: float) -> float:
    return add(x, -y)


def fma(x: float, y: float, z: float) -> float:
    p = Fraction(x) * Fraction(y)
    r = p + Fraction(z)
    if r == 0:
        p_neg = _neg0(x) != _neg0(y)
        both_zero = p == 0 and z == 0
        return -0.0 if (both_zero and p_neg and _neg0(z)) else 0.0
    return _round(r)


def to_f32(x) -> float:
    return _round(Fraction(float(x)))


def dot(x, y):
    """16 contiguous leaves (product, then fma ascending); pairwise sum of leaves."""
    d = len(x)
    m = d // 16
    leaves = []
    for l in range(16):
        acc = mul(x[l * m], y[l * m])
        for e in range(l * m + 1, l * m + m):
            acc = fma(x[e], y[e], acc)
        leaves.append(acc)
    width = 1
    while width < 16:
        for l in range(0, 16, 2 * width):
            leaves[l] = add(leaves[l], leaves[l + width])
        width *= 2
    return leaves[0]


def token(s, a, b, v_i, k, q):
    """One token on one state row; returns (new row, o_i)."""
    x = [mul(a, se) for se in s]
    u = dot(x, k)
    delta = mul(b, sub(v_i, u))
    s_new = [fma(delta, ke, xe) for ke, xe in zip(k, x)]
    return s_new, dot(s_new, q)


def row_tree(vals):
    """Pairwise tree over rows in natural order; a pair with no second half passes through."""
    vals = list(vals)
    n = len(vals)
    w = 1
    while w < n:
        for j in range(0, n - w, 2 * w):
            vals[j] = add(vals[j], vals[j + w])
        w *= 2
    return vals[0]


def backward(cu, q, k, v, a, b, do, s0, dsf, Hk):
    """The backward contract on tiny inputs (nested lists of binary32 Python floats).

    q, k [T][Hk][d]; v [T][Hv][dv]; a, b [T][Hv]; do [T][Hv][dv]; s0, dsf [N][Hv][dv][d].
    Returns dict dq, dk, dv, da, db, dS0 with the same nesting.
    """
    T = len(q)
    Hv = len(v[0])
    dv = len(v[0][0])
    d = len(q[0][0])
    G = Hv // Hk
    N = len(cu) - 1
    out = {"dq": [[[0.0] * d for _ in range(Hk)] for _ in range(T)],
           "dk": [[[0.0] * d for _ in range(Hk)] for _ in range(T)],
           "dv": [[[0.0] * dv for _ in range(Hv)] for _ in range(T)],
           "da": [[0.0] * Hv for _ in range(T)], "db": [[0.0] * Hv for _ in range(T)],
           "dS0": [[[None] * dv for _ in range(Hv)] for _ in range(N)]}
    for n in range(N):
        bos, eos = cu[n], cu[n + 1]
        for hk in range(Hk):
            dqh = [[[0.0] * d for _ in range(T)] for _ in range(G)]
            dkh = [[[0.0] * d for _ in range(T)] for _ in range(G)]
            for g in range(G):
                h = hk * G + g
                # forward states s_{t} for t = bos-1 .. eos-1, per row
                states = [[list(s0[n][h][i]) for i in range(dv)]]
                fwd = []
                for t in range(bos, eos):
                    cur, info = [], []
                    for i in range(dv):
                        s = states[-1][i]
                        x = [mul(a[t][h], se) for se in s]
                        u = dot(x, k[t][hk])
                        diff = sub(v[t][h][i], u)
                        delta = mul(b[t][h], diff)
                        cur.append([fma(delta, ke, xe) for ke, xe in zip(k[t][hk], x)])
                        info.append((x, diff, delta))
                    states.append(cur)
                    fwd.append(info)
                sh = [list(dsf[n][h][i]) for i in range(dv)]
                for t in range(eos - 1, bos - 1, -1):
                    j = t - bos
                    pq, pk, pa, pb = [], [], [], []
                    for i in range(dv):
                        x, diff, delta = fwd[j][i]
                        s_prev, s_cur = states[j][i], states[j + 1][i]
                        gg = do[t][h][i]
                        shr = [fma(gg, qe, se) for qe, se in zip(q[t][hk], sh[i])]
                        pq.append([mul(gg, se) for se in s_cur])
                        dh = dot(shr, k[t][hk])
                        dvi = mul(b[t][h], dh)
                        out["dv"][t][h][i] = dvi
                        pb.append(mul(dh, diff))
                        uh = -dvi
                        xh = [fma(uh, ke, se) for ke, se in zip(k[t][hk], shr)]
                        pk.append([fma(uh, xe, mul(delta, se)) for xe, se in zip(x, shr)])
                        pa.append(dot(xh, s_prev))
                        sh[i] = [mul(a[t][h], xe) for xe in xh]
                    out["da"][t][h] = row_tree(pa)
                    out["db"][t][h] = row_tree(pb)
                    dqh[g][j] = [row_tree([pq[i][e] for i in range(dv)]) for e in range(d)]
                    dkh[g][j] = [row_tree([pk[i][e] for i in range(dv)]) for e in range(d)]
                for i in range(dv):
                    out["dS0"][n][h][i] = sh[i]
            for t in range(bos, eos):
                for e in range(d):
                    aq, ak = dqh[0][t - bos][e], dkh[0][t - bos][e]
                    for g in range(1, G):
                        aq = add(aq, dqh[g][t - bos][e])
                        ak = add(ak, dkh[g][t - bos][e])
                    out["dq"][t][hk][e] = aq
                    out["dk"][t][hk][e] = ak
    return out


def cpr2_scan(cu, q, k, v, a, b, s0, chunk, Hk):
    """Two-level CPR on tiny inputs (nested lists of binary32 Python floats): transitions by
    the row update from unit rows (v = +0) and from zero rows, boundary states as fused
    multiply-adds in ascending k from B, outputs from rows restarted at every boundary.
    Returns (o [T][Hv][dv], chunk states [list of [Hv][dv][d]], final [N][Hv][dv][d])."""
    T, Hv, dv, d = len(q), len(v[0]), len(v[0][0]), len(q[0][0])
    G = Hv // Hk
    N = len(cu) - 1
    o = [[[0.0] * dv for _ in range(Hv)] for _ in range(T)]
    final = [[None] * Hv for _ in range(N)]
    states = []

    def absorb(s, at, bt, vi, kt):
        x = [mul(at, se) for se in s]
        u = dot(x, kt)
        delta = mul(bt, sub(vi, u))
        return [fma(delta, ke, xe) for ke, xe in zip(kt, x)]

    per_seq_states = []
    for n in range(N):
        bos, eos = cu[n], cu[n + 1]
        seq_states = []
        for h in range(Hv):
            hk = h // G
            S = [list(s0[n][h][i]) for i in range(dv)]
            R = [list(r) for r in S]
            hs = []
            for t0 in range(bos, eos, chunk):
                t1 = min(t0 + chunk, eos)
                R = [list(r) for r in S]
                for t in range(t0, t1):
                    for i in range(dv):
                        R[i], o[t][h][i] = token(R[i], a[t][h], b[t][h], v[t][h][i], k[t][hk],
                                                 q[t][hk])
                if t1 - t0 == chunk:
                    A = [[1.0 if j == e else 0.0 for e in range(d)] for j in range(d)]
                    B = [[0.0] * d for _ in range(dv)]
                    for t in range(t0, t1):
                        A = [absorb(A[j], a[t][h], b[t][h], 0.0, k[t][hk]) for j in range(d)]
                        B = [absorb(B[i], a[t][h], b[t][h], v[t][h][i], k[t][hk])
                             for i in range(dv)]
                    Sn = []
                    for i in range(dv):
                        row = []
                        for j in range(d):
                            acc = B[i][j]
                            for kk in range(d):
                                acc = fma(S[i][kk], A[kk][j], acc)
                            row.append(acc)
                        Sn.append(row)
                    S = Sn
                    hs.append([list(r) for r in S])
            final[n][h] = S if (eos - bos) % chunk == 0 else R
            seq_states.append(hs)
        per_seq_states.append(seq_states)
    for n in range(N):
        for c in range(len(per_seq_states[n][0]) if per_seq_states[n] else 0):
            states.append([per_seq_states[n][h][c] for h in range(Hv)])
    return o, states, final
