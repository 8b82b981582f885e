"""Pins of the CPU oracle against things other than itself.

Each ``pin_*`` takes an :class:`oracle.oracle.Oracle` and raises AssertionError when the
oracle disagrees with what the mathematics or a hand derivation fixes:
  * hand-derived reduction-order values (tests/golden/tree_order.json);
  * a dense float64 brute force of the gated delta rule (norm-wise relative error 1e-5);
  * exact closed forms with one-hot keys and queries, a in {1, 1/2}, b in {0, 1};
  * invariants: b=0 and a=1 leave S unchanged; unit k with b=1 makes S k = v;
  * an exact-rational binary32 emulator of the stated operation order (bitwise);
  * structural identities of the three cases (resume, chunk states, decode, packing);
  * for the linear region: the inner-product error bound against float64, the exact
    emulator, one-hot rows and batch invariance;
  * for the two-level CPR reading: the canonical bits when no chunk completes, float64,
    the exact emulator, identity transitions, decode with resync equal to the scan.
The same pins run against deliberately broken builds of the oracle (test_oracle_mutants),
which must each fail at least one of them.
"""

import json
import os

import numpy as np

import brute_f64
import exact_fp32
from bitwise_consistent_linear_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
REL_TOL_F64 = 1e-5


def _bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def same_bits(x, y) -> bool:
    x, y = np.asarray(x, np.float32), np.asarray(y, np.float32)
    return x.shape == y.shape and np.array_equal(_bits(x), _bits(y))


def _hexf(h):
    return np.uint32(int(h, 16)).view(np.float32)


def _vec(spec, d):
    if spec == "ones":
        return np.ones(d, np.float32)
    if spec == "zeros":
        return np.zeros(d, np.float32)
    if isinstance(spec, str) and spec.startswith("all "):
        return np.full(d, _hexf(spec[4:]), np.float32)
    out = np.zeros(d, np.float32)
    for i, h in spec.items():
        out[int(i)] = _hexf(h)
    return out


def _normwise(err_num, ref):
    den = np.abs(ref).max()
    return np.abs(err_num).max() / (den if den > 0 else 1.0)


def _check_f64(o, cs, fs, o64, cs64, fs64, cu, label):
    N = len(cu) - 1
    Hv = o.shape[1]
    for n in range(N):
        sl = slice(int(cu[n]), int(cu[n + 1]))
        for h in range(Hv):
            if sl.stop > sl.start:
                e = _normwise(o[sl, h] - o64[sl, h], o64[sl, h])
                assert e <= REL_TOL_F64, f"{label}: o rel err {e:.3g} at n={n} h={h}"
            e = _normwise(fs[n, h] - fs64[n, h], fs64[n, h])
            assert e <= REL_TOL_F64, f"{label}: final state rel err {e:.3g} at n={n} h={h}"
    assert cs.shape == cs64.shape, f"{label}: chunk state count {cs.shape} vs {cs64.shape}"
    for c in range(cs.shape[0]):
        e = _normwise(cs[c] - cs64[c], cs64[c])
        assert e <= REL_TOL_F64, f"{label}: chunk state {c} rel err {e:.3g}"


def small_case(seed, lengths, Hk, Hv, d, chunk, bf16=False, a_lo=0.9, with_s0=False):
    w = W.make_packed(f"small{seed}", lengths, Hk=Hk, Hv=Hv, d=d, chunk=chunk, bf16=bf16,
                      seed=1000 + seed, a_lo=a_lo)
    s0 = None
    if with_s0:
        g = np.random.default_rng(2000 + seed)
        s0 = (0.1 * g.standard_normal((w.num_seqs, Hv, d, d))).astype(np.float32)
    return w, s0


# ------------------------------------------------------------------------------ pins

def pin_tree_golden(orc):
    with open(os.path.join(GOLDEN, "tree_order.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x, y = _vec(c["x"], c["d"]), _vec(c["y"], c["d"])
        got = orc.dot(x, y)
        want = _hexf(c["expect"])
        assert same_bits(got, want), f"{c['name']}: got {got!r} want {want!r}"


def pin_dot_exact_emulator(orc):
    g = np.random.default_rng(11)
    for d in (16, 32, 64, 128):
        for _ in range(25):
            x = g.standard_normal(d).astype(np.float32) * np.float32(g.uniform(1e-3, 1e3))
            y = g.standard_normal(d).astype(np.float32)
            want = exact_fp32.dot([float(v) for v in x], [float(v) for v in y])
            got = orc.dot(x, y)
            assert same_bits(got, np.float32(want)), f"dot d={d}: {got!r} vs {want!r}"


def pin_tiny_vs_f64(orc):
    w = W.tiny()
    o, cs, fs = orc.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=w.chunk,
                         want_chunk_states=True, want_final_state=True)
    o64, cs64, fs64 = brute_f64.scan_f64(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, w.chunk)
    _check_f64(o, cs, fs, o64, cs64, fs64, w.cu_seqlens, "tiny")


def pin_shapes_vs_f64(orc):
    cases = [
        dict(seed=1, lengths=[5, 0, 37, 16], Hk=1, Hv=2, d=16, chunk=16),
        dict(seed=2, lengths=[23, 40], Hk=2, Hv=4, d=32, chunk=8, bf16=True),
        dict(seed=3, lengths=[33], Hk=2, Hv=2, d=64, chunk=16, with_s0=True),
        dict(seed=4, lengths=[7, 9, 18], Hk=1, Hv=4, d=16, chunk=4, bf16=True, with_s0=True),
    ]
    for c in cases:
        w, s0 = small_case(**c)
        o, cs, fs = orc.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=w.chunk,
                             initial_state=s0, want_chunk_states=True, want_final_state=True)
        o64, cs64, fs64 = brute_f64.scan_f64(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, w.chunk, s0)
        _check_f64(o, cs, fs, o64, cs64, fs64, w.cu_seqlens, f"case{c['seed']}")


def onehot_case(T=12, Hk=2, Hv=4, d=16, seed=5):
    g = np.random.default_rng(seed)
    kap = g.integers(0, d, (T, Hk))
    rho = g.integers(0, d, (T, Hk))
    q = np.zeros((T, Hk, d), np.float32)
    k = np.zeros((T, Hk, d), np.float32)
    for t in range(T):
        for j in range(Hk):
            k[t, j, kap[t, j]] = 1.0
            q[t, j, rho[t, j]] = 1.0
    v = g.integers(-8, 9, (T, Hv, d)).astype(np.float32)
    a = g.choice(np.float32([1.0, 0.5]), (T, Hv))
    b = g.choice(np.float32([0.0, 1.0]), (T, Hv))
    s0 = g.integers(-4, 5, (1, Hv, d, d)).astype(np.float32)
    return np.array([0, T], np.int32), q, k, v, a, b, s0, kap, rho


def pin_onehot_closed_form(orc):
    cu, q, k, v, a, b, s0, kap, rho = onehot_case()
    T, Hk, d = k.shape
    Hv = v.shape[1]
    G = Hv // Hk
    o, cs, fs = orc.scan(cu, q, k, v, a, b, chunk=4, initial_state=s0,
                         want_chunk_states=True, want_final_state=True)
    # closed form: column kappa of S becomes b*v + (1-b)*a*S[:, kappa]; other columns a*S
    S = s0[0].astype(np.float64).copy()
    for t in range(T):
        for h in range(Hv):
            kc, rc = kap[t, h // G], rho[t, h // G]
            S[h] *= float(a[t, h])
            if b[t, h] == 1.0:
                S[h][:, kc] = v[t, h]
            want_o = S[h][:, rc]
            assert np.array_equal(o[t, h].astype(np.float64), want_o), f"onehot o t={t} h={h}"
        if (t + 1) % 4 == 0:
            assert np.array_equal(cs[(t + 1) // 4 - 1].astype(np.float64), S), f"onehot chunk t={t}"
    assert np.array_equal(fs[0].astype(np.float64), S), "onehot final state"


def pin_b0_a1_identity(orc):
    w, _ = small_case(6, [20], Hk=2, Hv=2, d=32, chunk=4)
    g = np.random.default_rng(6)
    s0 = g.standard_normal((1, 2, 32, 32)).astype(np.float32)
    a = np.ones_like(w.a)
    b = np.zeros_like(w.b)
    o, cs, fs = orc.scan(w.cu_seqlens, w.q, w.k, w.v, a, b, chunk=4, initial_state=s0,
                         want_chunk_states=True, want_final_state=True)
    assert np.array_equal(fs, s0), "b=0, a=1 must leave the state unchanged"
    assert all(np.array_equal(cs[c], s0[0]) for c in range(cs.shape[0])), "chunk states changed"
    for t in range(20):
        for h in range(2):
            for i in range(32):
                want = exact_fp32.dot([float(x) for x in s0[0, h, i]],
                                      [float(x) for x in w.q[t, h]])
                assert same_bits(o[t, h, i], np.float32(want)), f"readout t={t} h={h} i={i}"


def pin_unit_k_overwrite(orc):
    # random unit k, b = 1: after every token S_t k_t = v_t up to rounding
    w, s0 = small_case(7, [16], Hk=1, Hv=2, d=64, chunk=16, with_s0=True)
    b = np.ones_like(w.b)
    k = w.k.astype(np.float64)
    for T in range(1, 17):
        cu = np.array([0, T], np.int32)
        _, _, fs = orc.scan(cu, w.q[:T], w.k[:T], w.v[:T], w.a[:T], b[:T], chunk=16,
                            initial_state=s0, want_o=False, want_final_state=True)
        for h in range(2):
            sk = fs[0, h].astype(np.float64) @ k[T - 1, 0]
            vt = w.v[T - 1, h].astype(np.float64)
            err = np.abs(sk - vt).max() / np.abs(vt).max()
            assert err <= 64 * 2.0 ** -22, f"unit k overwrite T={T} h={h}: rel {err:.3g}"


def pin_exact_emulator_tiny(orc):
    w = W.tiny()
    T = 24
    cu = np.array([0, T], np.int32)
    o, _, fs = orc.scan(cu, w.q[:T], w.k[:T], w.v[:T], w.a[:T], w.b[:T], chunk=16,
                        want_final_state=True)
    for h in range(w.num_v_heads):
        for i in range(0, w.d_v, 3):
            s = [0.0] * w.d_k
            for t in range(T):
                s, oi = exact_fp32.token(s, float(w.a[t, h]), float(w.b[t, h]),
                                         float(w.v[t, h, i]), [float(x) for x in w.k[t, h]],
                                         [float(x) for x in w.q[t, h]])
                assert same_bits(o[t, h, i], np.float32(oi)), f"emulator o t={t} h={h} i={i}"
            assert same_bits(fs[0, h, i], np.float32(s)), f"emulator state h={h} i={i}"


def pin_chunk_invariance(orc):
    w, s0 = small_case(8, [70, 33], Hk=1, Hv=2, d=16, chunk=16, with_s0=True)
    ref = None
    for C in (1, 4, 16, 64):
        o, _, fs = orc.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=C, initial_state=s0,
                            want_final_state=True)
        if ref is None:
            ref = (o, fs)
        assert same_bits(o, ref[0]) and same_bits(fs, ref[1]), f"C={C} changed o or state"


def pin_split_resume(orc):
    w, s0 = small_case(9, [50], Hk=2, Hv=2, d=32, chunk=8, bf16=True, with_s0=True)
    o, _, fs = orc.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=8, initial_state=s0,
                        want_final_state=True)
    for m in (1, 8, 21, 49):
        c1 = np.array([0, m], np.int32)
        c2 = np.array([0, 50 - m], np.int32)
        o1, _, f1 = orc.scan(c1, w.q[:m], w.k[:m], w.v[:m], w.a[:m], w.b[:m], chunk=8,
                             initial_state=s0, want_final_state=True)
        o2, _, f2 = orc.scan(c2, w.q[m:], w.k[m:], w.v[m:], w.a[m:], w.b[m:], chunk=8,
                             initial_state=f1, want_final_state=True)
        assert same_bits(np.concatenate([o1, o2]), o), f"split at {m}: o differs"
        assert same_bits(f2, fs), f"split at {m}: state differs"


def pin_chunk_states_are_prefix_finals(orc):
    w, s0 = small_case(10, [37, 16, 3], Hk=1, Hv=2, d=16, chunk=8, with_s0=True)
    _, cs, _ = orc.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=8, initial_state=s0,
                        want_o=False, want_chunk_states=True)
    c = 0
    for n, L in enumerate(w.lengths):
        bos = int(w.cu_seqlens[n])
        for j in range(8, int(L) + 1, 8):
            cu = np.array([0, j], np.int32)
            sl = slice(bos, bos + j)
            _, _, f = orc.scan(cu, w.q[sl], w.k[sl], w.v[sl], w.a[sl], w.b[sl], chunk=8,
                               initial_state=s0[n:n + 1], want_o=False, want_final_state=True)
            assert same_bits(cs[c], f[0]), f"chunk state {c} (n={n}, j={j})"
            c += 1
    assert c == cs.shape[0]


def pin_decode_equals_scan(orc):
    w, s0 = small_case(12, [40, 40, 40], Hk=2, Hv=4, d=32, chunk=8, bf16=True, with_s0=True)
    o, cs, fs = orc.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=8, initial_state=s0,
                         want_chunk_states=True, want_final_state=True)
    pre, steps = W.split_for_decode(w, 13)
    _, _, state = orc.scan(pre.cu_seqlens, pre.q, pre.k, pre.v, pre.a, pre.b, chunk=8,
                           initial_state=s0, want_o=False, want_final_state=True)
    o_seq = o.reshape(3, 40, 4, 32)
    cs_seq = cs.reshape(3, 5, 4, 32, 32)
    for s in range(27):
        od, rs = orc.decode_step(steps["pos"][s], steps["q"][s], steps["k"][s], steps["v"][s],
                                 steps["a"][s], steps["b"][s], state, chunk=8)
        assert same_bits(od, o_seq[:, 13 + s]), f"decode o at step {s}"
        if (13 + s + 1) % 8 == 0:
            assert same_bits(rs, cs_seq[:, (13 + s + 1) // 8 - 1]), f"resync at step {s}"
        else:
            assert not rs.any(), f"resync written off-boundary at step {s}"
    assert same_bits(state, fs), "decode end state"


def pin_permutation(orc):
    w, s0 = small_case(13, [9, 30, 17, 1], Hk=1, Hv=2, d=16, chunk=4, with_s0=True)
    o, cs, fs = orc.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=4, initial_state=s0,
                         want_chunk_states=True, want_final_state=True)
    perm = [2, 0, 3, 1]
    L = w.lengths
    idx = np.concatenate([np.arange(w.cu_seqlens[n], w.cu_seqlens[n + 1]) for n in perm])
    cu2 = np.concatenate([[0], np.cumsum(L[perm])]).astype(np.int32)
    o2, cs2, fs2 = orc.scan(cu2, w.q[idx], w.k[idx], w.v[idx], w.a[idx], w.b[idx], chunk=4,
                            initial_state=s0[perm], want_chunk_states=True,
                            want_final_state=True)
    assert same_bits(o2, o[idx]), "permuted pack: o"
    assert same_bits(fs2, fs[perm]), "permuted pack: final states"
    coff = np.concatenate([[0], np.cumsum(L // 4)])
    cidx = np.concatenate([np.arange(coff[n], coff[n + 1]) for n in perm]).astype(int)
    assert same_bits(cs2, cs[cidx]), "permuted pack: chunk states"


def pin_pairs_equals_full(orc):
    w, s0 = small_case(14, [19, 45], Hk=2, Hv=4, d=32, chunk=8, bf16=True, with_s0=True)
    o, cs, fs = orc.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=8, initial_state=s0,
                         want_chunk_states=True, want_final_state=True)
    pairs = [(1, 3), (0, 0), (1, 1)]
    res = orc.scan_pairs(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, pairs, chunk=8,
                         initial_state=s0)
    coff = np.concatenate([[0], np.cumsum(w.lengths // 8)])
    for (n, h), r in zip(pairs, res):
        sl = slice(int(w.cu_seqlens[n]), int(w.cu_seqlens[n + 1]))
        assert same_bits(r["o"], o[sl, h]), f"pair ({n},{h}) o"
        assert same_bits(r["chunk_states"], cs[coff[n]:coff[n + 1], h]), f"pair ({n},{h}) chunks"
        assert same_bits(r["final_state"], fs[n, h]), f"pair ({n},{h}) final"


def pin_idle_slot(orc):
    w, s0 = small_case(15, [4, 4], Hk=1, Hv=2, d=16, chunk=4, with_s0=True)
    state = s0.copy()
    pos = np.array([-1, 3], np.int32)
    q = w.q.reshape(2, 4, 1, 16)[:, 0]
    k = w.k.reshape(2, 4, 1, 16)[:, 0]
    v = w.v.reshape(2, 4, 2, 16)[:, 0]
    a = w.a.reshape(2, 4, 2)[:, 0]
    b = w.b.reshape(2, 4, 2)[:, 0]
    o, rs = orc.decode_step(pos, q, k, v, a, b, state, chunk=4)
    assert same_bits(state[0], s0[0]), "idle slot state changed"
    assert not o[0].any() and not rs[0].any(), "idle slot wrote outputs"
    assert not same_bits(state[1], s0[1]) and same_bits(rs[1], state[1]), "active slot resync"




# --------------------------------------------------------------------------- backward

GRAD_KEYS = ("dq", "dk", "dv", "da", "db", "dS0")


def bwd_case(seed, lengths, Hk, Hv, d, chunk=16, bf16=False):
    w, s0 = small_case(seed, lengths, Hk=Hk, Hv=Hv, d=d, chunk=chunk, bf16=bf16, with_s0=True)
    g = np.random.default_rng(3000 + seed)
    do = g.standard_normal((w.total_tokens, Hv, d)).astype(np.float32)
    dsf = (0.5 * g.standard_normal((w.num_seqs, Hv, d, d))).astype(np.float32)
    return w, s0, do, dsf


def pin_bwd_vs_autograd_f64(orc):
    for c in [(31, [37, 20], 1, 2, 32), (32, [64], 2, 4, 16), (33, [5, 0, 40], 1, 1, 64),
              (34, [29, 11], 1, 3, 16, 16, True)]:
        w, s0, do, dsf = bwd_case(*c)
        got = orc.backward(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, do, chunk=16,
                           initial_state=s0, dstate_final=dsf)
        ref = brute_f64.grads_torch_f64(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, s0, do, dsf)
        for key in GRAD_KEYS:
            e = _normwise(got[key].astype(np.float64) - ref[key], ref[key])
            assert e <= REL_TOL_F64, f"backward case {c[0]}: {key} rel err {e:.3g}"


def pin_bwd_finite_differences(orc):
    # directional derivatives of the float64 dense loss (no torch, no tree, no fmaf)
    w, s0, do, dsf = bwd_case(35, [9, 6], 1, 2, 16)
    got = orc.backward(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, do, chunk=16, initial_state=s0,
                       dstate_final=dsf)
    g = np.random.default_rng(35)
    base = {"q": w.q.astype(np.float64), "k": w.k.astype(np.float64),
            "v": w.v.astype(np.float64), "a": w.a.astype(np.float64),
            "b": w.b.astype(np.float64), "s0": s0.astype(np.float64)}
    names = {"q": "dq", "k": "dk", "v": "dv", "a": "da", "b": "db", "s0": "dS0"}
    for name, key in names.items():
        direction = g.standard_normal(base[name].shape)
        eps = 1e-6
        args = dict(base)
        args[name] = base[name] + eps * direction
        lp = brute_f64.loss_f64(w.cu_seqlens, args["q"], args["k"], args["v"], args["a"],
                                args["b"], args["s0"], do, dsf)
        args[name] = base[name] - eps * direction
        lm = brute_f64.loss_f64(w.cu_seqlens, args["q"], args["k"], args["v"], args["a"],
                                args["b"], args["s0"], do, dsf)
        fd = (lp - lm) / (2 * eps)
        an = float(np.sum(got[key].astype(np.float64) * direction))
        assert abs(fd - an) <= 1e-5 * max(1.0, abs(fd)), f"{key}: fd {fd:.9g} vs {an:.9g}"


def pin_bwd_exact_emulator(orc):
    # 5 rows (a ragged row tree), a group of 3 value heads (order of the group sum), C < T
    w, s0, do, dsf = bwd_case(36, [6, 3], 1, 3, 16)
    w.v = W.make_packed("v5", [6, 3], Hk=3, Hv=3, d=5, chunk=16, bf16=False, seed=36).v
    g = np.random.default_rng(36)
    s0 = (0.3 * g.standard_normal((2, 3, 5, 16))).astype(np.float32)
    do = g.standard_normal((9, 3, 5)).astype(np.float32)
    dsf = (0.5 * g.standard_normal((2, 3, 5, 16))).astype(np.float32)
    got = orc.backward(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, do, chunk=4, initial_state=s0,
                       dstate_final=dsf)
    tl = lambda x: np.asarray(x, np.float64).tolist()  # noqa: E731
    want = exact_fp32.backward([int(c) for c in w.cu_seqlens], tl(w.q), tl(w.k), tl(w.v),
                               tl(w.a), tl(w.b), tl(do), tl(s0), tl(dsf), Hk=1)
    for key in GRAD_KEYS:
        assert same_bits(got[key], np.array(want[key], np.float32)), f"emulator {key}"


def pin_bwd_linear_scaling(orc):
    # every gradient is linear in (do, dS_final): doubling both doubles every bit pattern
    w, s0, do, dsf = bwd_case(37, [21, 14], 2, 4, 32, chunk=8, bf16=True)
    r1 = orc.backward(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, do, chunk=8, initial_state=s0,
                      dstate_final=dsf)
    r2 = orc.backward(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, 2 * do, chunk=8, initial_state=s0,
                      dstate_final=2 * dsf)
    for key in GRAD_KEYS:
        assert same_bits(r2[key], 2 * r1[key]), f"scaling {key}"


def pin_bwd_chunk_invariance(orc):
    w, s0, do, dsf = bwd_case(38, [33, 17], 1, 2, 16)
    ref = None
    for C in (1, 4, 16, 64):
        r = orc.backward(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, do, chunk=C, initial_state=s0,
                         dstate_final=dsf)
        if ref is None:
            ref = r
        for key in GRAD_KEYS:
            assert same_bits(r[key], ref[key]), f"C={C} changed {key}"


# ------------------------------------------------------------------------ two-level CPR

def pin_cpr2_single_chunk_is_canonical(orc):
    # with no full chunk, the rows never leave the recurrence from S0: same bits as the
    # token-serial contract, outputs and final state alike
    w, s0 = small_case(51, [37, 0, 5, 63], Hk=2, Hv=4, d=32, chunk=64, bf16=True, with_s0=True)
    o, cs, fs = orc.cpr2_scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=64, initial_state=s0)
    ro, _, rfs = orc.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=64, initial_state=s0,
                          want_chunk_states=True, want_final_state=True)
    assert cs.shape[0] == 0, "no chunk state expected"
    assert same_bits(o, ro) and same_bits(fs, rfs), "single partial chunk differs from canonical"


def pin_cpr2_vs_f64(orc):
    # the two-level reading is the same mathematics: within the f64 tolerance
    for seed, lengths, Hk, Hv, d, C, bf16 in [(52, [50, 16, 7], 1, 2, 32, 16, False),
                                              (53, [64, 33], 2, 4, 16, 8, True),
                                              (54, [96], 1, 1, 64, 32, True)]:
        w, s0 = small_case(seed, lengths, Hk=Hk, Hv=Hv, d=d, chunk=C, bf16=bf16, with_s0=True)
        o, cs, fs = orc.cpr2_scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=C,
                                  initial_state=s0)
        o64, cs64, fs64 = brute_f64.scan_f64(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, C, s0)
        _check_f64(o, cs, fs, o64, cs64, fs64, w.cu_seqlens, f"cpr2 case {seed}")


def pin_cpr2_exact_emulator(orc):
    # 3 rows, C = 2, sequences of 5 (a tail) and 4 (ends on a boundary), two value heads
    w, s0 = small_case(55, [5, 4], Hk=1, Hv=2, d=16, chunk=2, with_s0=True)
    w.v = W.make_packed("v3", [5, 4], Hk=2, Hv=2, d=3, chunk=2, bf16=False, seed=55).v
    s0 = (0.3 * np.random.default_rng(55).standard_normal((2, 2, 3, 16))).astype(np.float32)
    o, cs, fs = orc.cpr2_scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=2, initial_state=s0)
    tl = lambda x: np.asarray(x, np.float64).tolist()  # noqa: E731
    eo, ecs, efs = exact_fp32.cpr2_scan([int(c) for c in w.cu_seqlens], tl(w.q), tl(w.k),
                                        tl(w.v), tl(w.a), tl(w.b), tl(s0), 2, Hk=1)
    assert same_bits(o, np.array(eo, np.float32)), "cpr2 outputs"
    assert same_bits(cs, np.array(ecs, np.float32)), "cpr2 chunk states"
    assert same_bits(fs, np.array(efs, np.float32)), "cpr2 final states"


def pin_cpr2_identity_transition(orc):
    # a = 1, b = 0: every transition is exactly the identity and B = 0, so every boundary
    # state equals S0 and every output is the contract dot of S0's row with q
    w, s0 = small_case(56, [24, 16], Hk=1, Hv=2, d=32, chunk=8, with_s0=True)
    w.a[:] = 1.0
    w.b[:] = 0.0
    s0[s0 == 0] = 0.5
    o, cs, fs = orc.cpr2_scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=8, initial_state=s0)
    ro, _, _ = orc.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=8, initial_state=s0,
                        want_chunk_states=True, want_final_state=True)
    assert same_bits(o, ro), "outputs with identity transitions"
    want = np.concatenate([np.repeat(s0[0:1], 3, 0), np.repeat(s0[1:2], 2, 0)])
    assert np.array_equal(cs, want) and np.array_equal(fs, s0), "boundary states moved"


def pin_cpr2_decode_equals_scan(orc):
    # token-by-token decode with resync from the cache gives the scan's bits: outputs, every
    # resync checkpoint, and the final state (sequences ending on and off a boundary)
    for T in (24, 27):
        w, s0 = small_case(57, [T, T], Hk=2, Hv=4, d=32, chunk=8, bf16=True, with_s0=True)
        o, cs, fs = orc.cpr2_scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=8,
                                  initial_state=s0)
        _, steps = W.split_for_decode(w, 0)
        dec = orc.cpr2_decoder(2, 2, 4, 32, 32, chunk=8, initial_state=s0)
        c = 0
        for t in range(T):
            od, rs = orc.cpr2_decode_step(dec, steps["pos"][t], steps["q"][t], steps["k"][t],
                                          steps["v"][t], steps["a"][t], steps["b"][t])
            assert same_bits(od, o.reshape(2, T, 4, 32)[:, t]), f"decode o at t={t}"
            if (t + 1) % 8 == 0:
                assert same_bits(rs[0], cs[c]) and same_bits(rs[1], cs[T // 8 + c]), "resync"
                c += 1
        assert same_bits(dec["state"], fs), f"decode final state T={T}"


# --------------------------------------------------------------------------- linear region

def _widen(a):
    a = np.asarray(a)
    return W.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a.astype(np.float32)


def linear_error_bound(x, w):
    """Forward error bound of the contract dot with leaves of m = K/16 elements: every
    product and partial sum passes through at most m + 4 roundings (m in a leaf, 4 tree
    levels), so |y - x.w| <= gamma_{m+4} * sum_k |x_k w_k| with gamma_n = n u / (1 - n u),
    u = 2^-24 (the standard inner-product bound, Higham, Accuracy and Stability of
    Numerical Algorithms, section 3.1)."""
    K = x.shape[1]
    n = K // 16 + 4
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    return gamma * (np.abs(_widen(x).astype(np.float64)) @ np.abs(_widen(w).astype(np.float64)))


def pin_linear_vs_f64(orc):
    for M, N, K, bf16, seed in [(17, 23, 512, True, 41), (9, 5, 96, False, 42), (3, 64, 4096, True, 43)]:
        x, w = W.make_linear(M, N, K, bf16, seed)
        y = orc.linear(x, w)
        y64 = _widen(x).astype(np.float64) @ _widen(w).astype(np.float64)
        err = np.abs(y.astype(np.float64) - y64)
        bound = linear_error_bound(x, w)
        assert np.all(err <= bound), f"linear ({M},{N},{K}): err exceeds the bound"
        assert err.max() > 0, "no rounding at all: suspicious"


def pin_linear_exact_emulator(orc):
    # spread exponents so that the leaf chains, the fused steps and the tree all round
    g = np.random.default_rng(44)
    for K in (16, 48):
        x = (g.standard_normal((3, K)) * 2.0 ** g.integers(-12, 12, (3, K))).astype(np.float32)
        w = (g.standard_normal((K, 4)) * 2.0 ** g.integers(-12, 12, (K, 4))).astype(np.float32)
        y = orc.linear(x, w)
        for m in range(3):
            for n in range(4):
                want = exact_fp32.dot([float(v) for v in x[m]], [float(v) for v in w[:, n]])
                assert same_bits(y[m, n], np.float32(want)), f"emulator K={K} ({m},{n})"


def pin_linear_onehot_rows(orc):
    # a one-hot row of x selects a row of w exactly: catches a transposed w or shifted rows
    K = N = 64
    g = np.random.default_rng(45)
    w = g.standard_normal((K, N)).astype(np.float32)
    w[w == 0] = 1.0
    picks = g.permutation(K)[:10]
    x = np.zeros((10, K), np.float32)
    x[np.arange(10), picks] = 1.0
    y = orc.linear(x, w)
    assert same_bits(y, w[picks]), "one-hot rows do not select the rows of w"


def pin_linear_batch_invariance(orc):
    # a row's output does not depend on the other rows or on the column split
    x, w = W.make_linear(40, 24, 256, True, 46)
    y = orc.linear(x, w)
    assert same_bits(orc.linear(x[13:14], w), y[13:14]), "single row differs"
    assert same_bits(orc.linear(x[5:29], w), y[5:29]), "row slice differs"
    assert same_bits(orc.linear(x, np.ascontiguousarray(w[:, 7:19])), y[:, 7:19]), "column slice"
    x2, _ = W.make_linear(7, 24, 256, True, 46)
    assert same_bits(x2, x[:7]), "the generator's rows are not a prefix"


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
