"""The C ABI on the host: exports, identity, claims. No GPU is touched: every call here is
refused by a host-side check before anything is enqueued (fake pointers are never read)."""

import ctypes
import hashlib
import json
import os
import re
import subprocess

import pytest

from bitwise_consistent_linear_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn_cpr.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

CHUNKS = (16, 32, 64, 128, 256)
DKS = (16, 32, 64, 128)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return api.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) == 18, names
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(gdn_\w+)$", out, flags=re.M))
    assert set(names) <= exported, set(names) - exported
    assert exported <= set(names), f"undeclared exports: {exported - set(names)}"
    for n in names:
        assert hasattr(L, n)


def test_abi_version_matches_header(L):
    m = re.search(r"#define GDN_CPR_ABI_VERSION (\d+)", open(HEADER).read())
    assert api.abi_version() == int(m.group(1))


@pytest.mark.parametrize("n", [0, 1, 3, 55, 56, 57, 63, 64, 65, 119, 120, 127, 128, 129, 1000])
def test_sha256_matches_hashlib(n):
    data = bytes((i * 131 + 7) % 256 for i in range(n))
    assert api.sha256(data) == hashlib.sha256(data).digest()


@pytest.mark.parametrize("chunk", CHUNKS)
@pytest.mark.parametrize("d_k", DKS)
def test_identity_is_sha256_of_contract_text(chunk, d_k):
    text = api.contract_string(chunk, d_k)
    assert f"chunk={chunk}\n" in text and f"d_k={d_k}\n" in text
    assert "leaves:16" in text and "fusion=explicit fma only" in text
    assert api.contract_identity(chunk, d_k) == hashlib.sha256(text.encode()).digest()


def test_identities_are_distinct():
    ids = {api.contract_identity(c, d) for c in CHUNKS for d in DKS}
    assert len(ids) == len(CHUNKS) * len(DKS)


@pytest.mark.parametrize("chunk", CHUNKS)
@pytest.mark.parametrize("d_k", DKS)
def test_contract_text_matches_the_written_spec(chunk, d_k):
    """tests/golden/contract_text.txt is the contract written out by hand; the library's
    text, and so its identity, must be exactly that text for every admitted (C, d_k)."""
    with open(os.path.join(GOLDEN, "contract_text.txt")) as f:
        want = f.read().replace("{chunk}", str(chunk)).replace("{d_k}", str(d_k))
    assert api.contract_string(chunk, d_k) == want
    assert api.contract_identity(chunk, d_k) == hashlib.sha256(want.encode()).digest()


@pytest.mark.parametrize("chunk,d_k", [(48, 128), (0, 128), (64, 48), (64, 256), (-16, 16)])
def test_unadmitted_contract_refused(L, chunk, d_k):
    buf = ctypes.create_string_buffer(32)
    assert L.gdn_contract_identity(chunk, d_k, buf) == api.GDN_E_UNSUPPORTED
    n = ctypes.c_size_t(0)
    assert L.gdn_contract_string(chunk, d_k, None, 0, ctypes.byref(n)) == api.GDN_E_UNSUPPORTED


def test_contract_string_small_buffer(L):
    n = ctypes.c_size_t(0)
    assert L.gdn_contract_string(64, 128, None, 0, ctypes.byref(n)) == api.GDN_E_SHAPE
    assert n.value == len(api.contract_string(64, 128))
    assert L.gdn_contract_string(64, 128, None, 0, None) == api.GDN_E_NULL


# ------------------------------------------------------------------- refused compute calls

FAKE = 0x100000  # never dereferenced: every call below is refused on the host


def shape(**kw):
    base = dict(num_seqs=2, num_qk_heads=2, num_v_heads=4, d_k=64, d_v=64, chunk=64,
                qkv_dtype=api.GDN_DTYPE_BF16)
    base.update(kw)
    return api.GdnShape(**base)


def ident(sh):
    if sh is None or sh.chunk not in CHUNKS or sh.d_k not in DKS:
        return bytes(32)
    return api.contract_identity(sh.chunk, sh.d_k)


def trainer(L, sh, identity=None, T=128, total_chunks=2, **ptrs):
    p = dict(cu=FAKE, q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, s0=None, o=FAKE, cs=FAKE)
    p.update(ptrs)
    idb = ident(sh) if identity is None else identity
    return L.gdn_cpr_trainer_fwd(ctypes.byref(sh) if sh is not None else None, idb, p["cu"], T,
                                 p["q"], p["k"], p["v"], p["a"], p["b"], p["s0"], p["o"],
                                 p["cs"], total_chunks, None)


def prefill(L, sh, identity=None, T=128, **ptrs):
    p = dict(cu=FAKE, q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, s0=None, o=FAKE, fs=FAKE)
    p.update(ptrs)
    idb = ident(sh) if identity is None else identity
    return L.gdn_cpr_prefill(ctypes.byref(sh), idb, p["cu"], T, p["q"], p["k"], p["v"],
                             p["a"], p["b"], p["s0"], p["o"], p["fs"], None)


def bwd(L, sh, identity=None, T=128, total_chunks=2, ws_bytes=1 << 30, **ptrs):
    p = dict(cu=FAKE, q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, s0=None, cs=FAKE, do=FAKE,
             dsf=None, dq=FAKE, dk=FAKE, dv=FAKE, da=FAKE, db=FAKE, ds0=FAKE, ws=FAKE)
    p.update(ptrs)
    idb = ident(sh) if identity is None else identity
    return L.gdn_cpr_trainer_bwd(ctypes.byref(sh), idb, p["cu"], T, p["q"], p["k"], p["v"],
                                 p["a"], p["b"], p["s0"], p["cs"], total_chunks, p["do"],
                                 p["dsf"], p["dq"], p["dk"], p["dv"], p["da"], p["db"],
                                 p["ds0"], p["ws"], ws_bytes, None)


def bwd_noalloc(L, sh, identity=None, T=128, total_chunks=2, **ptrs):
    p = dict(cu=FAKE, q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, s0=None, cs=FAKE, do=FAKE,
             dsf=None, dq=FAKE, dk=FAKE, dv=FAKE, da=FAKE, db=FAKE, ds0=FAKE)
    p.update(ptrs)
    idb = ident(sh) if identity is None else identity
    return L.gdn_cpr_trainer_bwd_noalloc(ctypes.byref(sh), idb, p["cu"], T, p["q"], p["k"],
                                         p["v"], p["a"], p["b"], p["s0"], p["cs"], total_chunks,
                                         p["do"], p["dsf"], p["dq"], p["dk"], p["dv"], p["da"],
                                         p["db"], p["ds0"], None)


def linear(L, m=64, n=64, k=512, xdt=api.GDN_DTYPE_BF16, wdt=api.GDN_DTYPE_BF16, identity=None,
           x=FAKE, w=FAKE, y=FAKE, shape_ok=True):
    sh = api.GdnLinearShape(m, n, k, xdt, wdt)
    idb = api.contract_identity(64, 128) if identity is None else identity
    return L.gdn_linear_fwd(ctypes.byref(sh) if shape_ok else None, idb, x, w, y, None)


def decode(L, sh, identity=None, **ptrs):
    p = dict(pos=FAKE, q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, state=FAKE, o=FAKE, rs=None)
    p.update(ptrs)
    idb = ident(sh) if identity is None else identity
    return L.gdn_cpr_decode_step(ctypes.byref(sh), idb, p["pos"], p["q"], p["k"], p["v"],
                                 p["a"], p["b"], p["state"], p["o"], p["rs"], None)


def cpr2_ident(sh):
    if sh is None or sh.chunk not in CHUNKS or sh.d_k not in DKS[1:]:
        return bytes(32)
    return api.cpr2_contract_identity(sh.chunk, sh.d_k)


def cpr2_batch(L, sh, prefill_case=False, identity=None, T=128, total_chunks=2,
               ws_bytes=1 << 30, **ptrs):
    p = dict(cu=FAKE, q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, s0=None, o=FAKE, out=FAKE,
             ws=FAKE)
    p.update(ptrs)
    idb = cpr2_ident(sh) if identity is None else identity
    fn = L.gdn_cpr2_prefill if prefill_case else L.gdn_cpr2_trainer_fwd
    return fn(ctypes.byref(sh), idb, p["cu"], T, p["q"], p["k"], p["v"], p["a"], p["b"],
              p["s0"], p["o"], p["out"], total_chunks, p["ws"], ws_bytes, None)


def cpr2_decode(L, sh, identity=None, ws_bytes=1 << 30, **ptrs):
    p = dict(pos=FAKE, q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, state=FAKE, bnd=FAKE,
             ck=FAKE, cv=FAKE, ca=FAKE, cb=FAKE, o=FAKE, rs=None, ws=FAKE)
    p.update(ptrs)
    idb = cpr2_ident(sh) if identity is None else identity
    return L.gdn_cpr2_decode_step(ctypes.byref(sh), idb, p["pos"], p["q"], p["k"], p["v"],
                                  p["a"], p["b"], p["state"], p["bnd"], p["ck"], p["cv"],
                                  p["ca"], p["cb"], p["o"], p["rs"], p["ws"], ws_bytes, None)


REFUSALS = [
    ("null shape", lambda L: trainer(L, None), api.GDN_E_NULL),
    ("null identity", lambda L: L.gdn_cpr_trainer_fwd(ctypes.byref(shape()), None, FAKE, 128, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 2, None), api.GDN_E_NULL),
    ("wrong identity", lambda L: trainer(L, shape(), identity=bytes(32)), api.GDN_E_IDENTITY),
    ("identity of other chunk", lambda L: trainer(L, shape(), identity=api.contract_identity(16, 64)), api.GDN_E_IDENTITY),
    ("identity of other d_k", lambda L: prefill(L, shape(), identity=api.contract_identity(64, 128)), api.GDN_E_IDENTITY),
    ("heads not a multiple", lambda L: trainer(L, shape(num_qk_heads=3, num_v_heads=4)), api.GDN_E_SHAPE),
    ("zero qk heads", lambda L: trainer(L, shape(num_qk_heads=0)), api.GDN_E_SHAPE),
    ("heads x width > 2^20", lambda L: trainer(L, shape(num_qk_heads=1, num_v_heads=16385)), api.GDN_E_SHAPE),
    ("negative seqs", lambda L: trainer(L, shape(num_seqs=-1)), api.GDN_E_SHAPE),
    ("d_k not admitted", lambda L: trainer(L, shape(d_k=48)), api.GDN_E_UNSUPPORTED),
    ("d_v zero", lambda L: trainer(L, shape(d_v=0)), api.GDN_E_UNSUPPORTED),
    ("d_v too large", lambda L: trainer(L, shape(d_v=1025)), api.GDN_E_UNSUPPORTED),
    ("chunk not admitted", lambda L: trainer(L, shape(chunk=48)), api.GDN_E_UNSUPPORTED),
    ("dtype not admitted", lambda L: trainer(L, shape(qkv_dtype=7)), api.GDN_E_UNSUPPORTED),
    ("negative tokens", lambda L: trainer(L, shape(), T=-1), api.GDN_E_SHAPE),
    ("tokens >= 2^31", lambda L: trainer(L, shape(), T=2**31), api.GDN_E_SHAPE),
    ("negative chunks", lambda L: trainer(L, shape(), total_chunks=-1), api.GDN_E_SHAPE),
    ("more chunks than T/C", lambda L: trainer(L, shape(), total_chunks=3), api.GDN_E_SHAPE),
    ("null cu_seqlens", lambda L: trainer(L, shape(), cu=None), api.GDN_E_NULL),
    ("null q", lambda L: trainer(L, shape(), q=None), api.GDN_E_NULL),
    ("null b", lambda L: prefill(L, shape(), b=None), api.GDN_E_NULL),
    ("null o", lambda L: trainer(L, shape(), o=None), api.GDN_E_NULL),
    ("null chunk_states", lambda L: trainer(L, shape(), cs=None), api.GDN_E_NULL),
    ("null final_state", lambda L: prefill(L, shape(), fs=None), api.GDN_E_NULL),
    ("misaligned q (bf16 needs 8 B)", lambda L: trainer(L, shape(), q=FAKE + 4), api.GDN_E_SHAPE),
    ("misaligned k (f32 needs 16 B)", lambda L: trainer(L, shape(qkv_dtype=api.GDN_DTYPE_F32), k=FAKE + 8), api.GDN_E_SHAPE),
    ("misaligned initial state", lambda L: prefill(L, shape(), s0=FAKE + 4), api.GDN_E_SHAPE),
    ("misaligned chunk states", lambda L: trainer(L, shape(), cs=FAKE + 8), api.GDN_E_SHAPE),
    ("decode null pos", lambda L: decode(L, shape(), pos=None), api.GDN_E_NULL),
    ("decode null state", lambda L: decode(L, shape(), state=None), api.GDN_E_NULL),
    ("decode null v", lambda L: decode(L, shape(), v=None), api.GDN_E_NULL),
    ("decode misaligned state", lambda L: decode(L, shape(), state=FAKE + 4), api.GDN_E_SHAPE),
    ("decode misaligned resync", lambda L: decode(L, shape(), rs=FAKE + 4), api.GDN_E_SHAPE),
    ("decode wrong identity", lambda L: decode(L, shape(), identity=b"\x01" * 32), api.GDN_E_IDENTITY),
    ("decode chunk not admitted", lambda L: decode(L, shape(chunk=100)), api.GDN_E_UNSUPPORTED),
    ("bwd wrong identity", lambda L: bwd(L, shape(), identity=bytes(32)), api.GDN_E_IDENTITY),
    ("bwd chunk not admitted", lambda L: bwd(L, shape(chunk=100), total_chunks=1), api.GDN_E_UNSUPPORTED),
    ("bwd chunk 8", lambda L: bwd(L, shape(chunk=8), total_chunks=0), api.GDN_E_UNSUPPORTED),
    ("bwd more chunks than T/C", lambda L: bwd(L, shape(), total_chunks=3), api.GDN_E_SHAPE),
    ("bwd null chunk_states", lambda L: bwd(L, shape(), cs=None), api.GDN_E_NULL),
    ("bwd null d_o", lambda L: bwd(L, shape(), do=None), api.GDN_E_NULL),
    ("bwd null dk", lambda L: bwd(L, shape(), dk=None), api.GDN_E_NULL),
    ("bwd null db", lambda L: bwd(L, shape(), db=None), api.GDN_E_NULL),
    ("bwd null dS0", lambda L: bwd(L, shape(), ds0=None), api.GDN_E_NULL),
    ("bwd null workspace", lambda L: bwd(L, shape(), ws=None), api.GDN_E_NULL),
    ("bwd misaligned workspace", lambda L: bwd(L, shape(), ws=FAKE + 64), api.GDN_E_SHAPE),
    ("bwd workspace too small", lambda L: bwd(L, shape(), ws_bytes=256), api.GDN_E_SHAPE),
    ("bwd misaligned d_final_state", lambda L: bwd(L, shape(), dsf=FAKE + 4), api.GDN_E_SHAPE),
    ("bwd misaligned dq", lambda L: bwd(L, shape(), dq=FAKE + 2), api.GDN_E_SHAPE),
    ("bwd null q", lambda L: bwd(L, shape(), q=None), api.GDN_E_NULL),
    ("bwd heads not a multiple", lambda L: bwd(L, shape(num_qk_heads=3)), api.GDN_E_SHAPE),
    ("bwd noalloc wrong identity", lambda L: bwd_noalloc(L, shape(), identity=bytes(32)), api.GDN_E_IDENTITY),
    ("bwd noalloc null d_o", lambda L: bwd_noalloc(L, shape(), do=None), api.GDN_E_NULL),
    # 2^20 tokens of 16 heads at d = 128 need gigabytes of workspace: more than the fixed array
    ("bwd noalloc beyond the fixed array", lambda L: bwd_noalloc(L, shape(num_seqs=1, num_qk_heads=16, num_v_heads=16, d_k=128, d_v=128), T=1 << 20, total_chunks=(1 << 20) // 64), api.GDN_E_SHAPE),
    ("cpr2 one-level identity", lambda L: cpr2_batch(L, shape(), identity=api.contract_identity(64, 64)), api.GDN_E_IDENTITY),
    ("one-level call, two-level identity", lambda L: trainer(L, shape(), identity=api.cpr2_contract_identity(64, 64)), api.GDN_E_IDENTITY),
    ("cpr2 d_k 16", lambda L: cpr2_batch(L, shape(d_k=16)), api.GDN_E_UNSUPPORTED),
    ("cpr2 more chunks than T/C", lambda L: cpr2_batch(L, shape(), total_chunks=3), api.GDN_E_SHAPE),
    ("cpr2 null chunk_states", lambda L: cpr2_batch(L, shape(), out=None), api.GDN_E_NULL),
    ("cpr2 null workspace", lambda L: cpr2_batch(L, shape(), ws=None), api.GDN_E_NULL),
    ("cpr2 misaligned workspace", lambda L: cpr2_batch(L, shape(), ws=FAKE + 16), api.GDN_E_SHAPE),
    ("cpr2 workspace too small", lambda L: cpr2_batch(L, shape(), ws_bytes=1024), api.GDN_E_SHAPE),
    ("cpr2 prefill null final", lambda L: cpr2_batch(L, shape(), True, out=None), api.GDN_E_NULL),
    ("cpr2 prefill final aliases initial", lambda L: cpr2_batch(L, shape(), True, s0=FAKE), api.GDN_E_SHAPE),
    ("cpr2 prefill null v", lambda L: cpr2_batch(L, shape(), True, v=None), api.GDN_E_NULL),
    ("cpr2 decode null boundary", lambda L: cpr2_decode(L, shape(), bnd=None), api.GDN_E_NULL),
    ("cpr2 decode null cache", lambda L: cpr2_decode(L, shape(), cv=None), api.GDN_E_NULL),
    ("cpr2 decode misaligned cache_k", lambda L: cpr2_decode(L, shape(), ck=FAKE + 8), api.GDN_E_SHAPE),
    ("cpr2 decode misaligned boundary", lambda L: cpr2_decode(L, shape(), bnd=FAKE + 4), api.GDN_E_SHAPE),
    ("cpr2 decode workspace too small", lambda L: cpr2_decode(L, shape(), ws_bytes=256), api.GDN_E_SHAPE),
    ("cpr2 decode one-level identity", lambda L: cpr2_decode(L, shape(), identity=api.contract_identity(64, 64)), api.GDN_E_IDENTITY),
    ("linear null shape", lambda L: linear(L, shape_ok=False), api.GDN_E_NULL),
    ("linear wrong identity", lambda L: linear(L, identity=bytes(32)), api.GDN_E_IDENTITY),
    ("linear k not a multiple of 512", lambda L: linear(L, k=768), api.GDN_E_UNSUPPORTED),
    ("linear k zero", lambda L: linear(L, k=0), api.GDN_E_UNSUPPORTED),
    ("linear dtype not admitted", lambda L: linear(L, xdt=5), api.GDN_E_UNSUPPORTED),
    ("linear negative m", lambda L: linear(L, m=-1), api.GDN_E_SHAPE),
    ("linear m too large", lambda L: linear(L, m=2**31), api.GDN_E_SHAPE),
    ("linear null x", lambda L: linear(L, x=None), api.GDN_E_NULL),
    ("linear null y", lambda L: linear(L, y=None), api.GDN_E_NULL),
    ("linear misaligned w", lambda L: linear(L, w=FAKE + 8), api.GDN_E_SHAPE),
]


@pytest.mark.parametrize("name,call,status", REFUSALS, ids=[r[0] for r in REFUSALS])
def test_refused_before_launch(L, name, call, status):
    assert call(L) == status
    msg = L.gdn_last_error().decode()
    assert msg.startswith(("gdn_cpr_", "gdn_cpr2_", "gdn_linear_")), msg


def test_binding_raises_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(api, "_lib", None)
    monkeypatch.setattr(api, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="missing"):
        api.lib()


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "bitwise_consistent_linear_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, flags=re.M), f
                assert "gdn_oracle" not in text and "liboracle" not in text, f


def test_bwd_workspace_size(L):
    """The workspace holds the plan, the chunk-boundary gradients and the row-block partial
    sums; it grows with tokens and chunks and is refused for unadmitted sizes."""
    sh = shape(num_seqs=3, num_v_heads=4, d_k=64, d_v=40, chunk=32)
    small = api.trainer_bwd_workspace_bytes(sh, 100, 2)
    big = api.trainer_bwd_workspace_bytes(sh, 1000, 30)
    rb = 2  # ceil(40 / 32) blocks of 32 rows
    assert small >= 100 * 4 * rb * (2 * 64 + 2) * 4 + 2 * 4 * 40 * 64 * 4
    assert big > small and small % 256 == 0 and big % 256 == 0
    n = ctypes.c_size_t(0)
    assert L.gdn_cpr_trainer_bwd_workspace(ctypes.byref(shape(chunk=100)), 128, 1,
                                           ctypes.byref(n)) == api.GDN_E_UNSUPPORTED
    for c in (128, 256):  # long chunks are admitted
        assert L.gdn_cpr_trainer_bwd_workspace(ctypes.byref(shape(chunk=c)), 300, 1,
                                               ctypes.byref(n)) == api.GDN_OK
    assert L.gdn_cpr_trainer_bwd_workspace(ctypes.byref(sh), 100, 4,
                                           ctypes.byref(n)) == api.GDN_E_SHAPE
    assert L.gdn_cpr_trainer_bwd_workspace(ctypes.byref(sh), 100, 2, None) == api.GDN_E_NULL


def test_linear_accepts_every_contract_identity_and_empty_sizes(L):
    """The linear rule is part of every contract text; m == 0 or n == 0 launches nothing
    (fake pointers are never touched)."""
    for c in CHUNKS:
        for d in DKS:
            assert linear(L, m=0, identity=api.contract_identity(c, d)) == api.GDN_OK
    assert linear(L, n=0, x=None, w=None, y=None) == api.GDN_OK


@pytest.mark.parametrize("chunk", CHUNKS)
@pytest.mark.parametrize("d_k", DKS[1:])
def test_two_level_contract_text(chunk, d_k):
    """The two-level text is the canonical text with its one-level "cpr=" line replaced by
    the two-level lines, and its identity is the SHA-256 of that text."""
    one = api.contract_string(chunk, d_k).splitlines(keepends=True)
    two = api.cpr2_contract_string(chunk, d_k)
    at = [i for i, line in enumerate(one) if line.startswith("cpr=")]
    assert len(at) == 1 and one[at[0]].startswith("cpr=one_level;")
    lines = two.splitlines(keepends=True)
    assert lines[:at[0]] == one[:at[0]] and lines[at[0]] == "cpr=two_level\n"
    extra = lines[at[0] + 1:len(lines) - (len(one) - at[0] - 1)]
    assert [x.split("=")[0] for x in extra] == [
        "two_level_transition", "two_level_boundary", "two_level_outputs", "two_level_final",
        "two_level_decode"]
    assert lines[len(lines) - (len(one) - at[0] - 1):] == one[at[0] + 1:]
    assert api.cpr2_contract_identity(chunk, d_k) == hashlib.sha256(two.encode()).digest()
    assert api.cpr2_contract_identity(chunk, d_k) != api.contract_identity(chunk, d_k)


def test_two_level_d_k_16_not_admitted(L):
    buf = ctypes.create_string_buffer(32)
    assert L.gdn_cpr2_contract_identity(64, 16, buf) == api.GDN_E_UNSUPPORTED


def test_cpr2_workspace_size(L):
    """Batch: the plan, chunk bases, one A_c [d_k, d_k] and B_c [d_v, d_k] per full chunk and
    head, and the prefill's boundary states; decode: one A_c and B_c per sequence and head."""
    sh = shape(num_seqs=3, num_v_heads=4, d_k=64, d_v=40, chunk=32)
    batch = api.cpr2_workspace_bytes(sh, 1000, 30, False)
    dec = api.cpr2_workspace_bytes(sh, 0, 0, True)
    assert batch >= 30 * 4 * (64 * 64 + 40 * 64) * 4 + 30 * 4 * 40 * 64 * 4
    assert dec >= 3 * 4 * (64 * 64 + 40 * 64) * 4
    assert batch % 256 == 0 and dec % 256 == 0
    n = ctypes.c_size_t(0)
    assert L.gdn_cpr2_workspace(ctypes.byref(sh), 100, 4, 0, ctypes.byref(n)) == api.GDN_E_SHAPE
    assert L.gdn_cpr2_workspace(ctypes.byref(sh), 100, 2, 0, None) == api.GDN_E_NULL
    assert L.gdn_cpr2_workspace(ctypes.byref(shape(d_k=16)), 0, 0, 1,
                                ctypes.byref(n)) == api.GDN_E_SHAPE


def test_linear_accepts_two_level_identities(L):
    for d in DKS[1:]:
        assert linear(L, m=0, identity=api.cpr2_contract_identity(64, d)) == api.GDN_OK
