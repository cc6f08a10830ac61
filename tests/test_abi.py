"""The C ABI without a GPU: the library loads, exports every function include/condensate.h
declares, and rejects bad arguments on the host before touching HIP."""
import ctypes
import os
import re

import pytest

import sparse_transformer_attention_amd as ca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "condensate.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ca_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ca.LIB_PATH):
        from sparse_transformer_attention_amd import build
        build.build(verbose=False)
    return ca.load()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(ca.EXPORTED)
    for name in names:
        assert hasattr(lib, name), f"{name} not exported"


def test_status_strings(lib):
    for rc in (ca.CA_OK, ca.CA_ERR_INVALID_ARG, ca.CA_ERR_UNSUPPORTED, ca.CA_ERR_WORKSPACE, ca.CA_ERR_HIP):
        s = ca.status_string(rc)
        assert s.startswith("CA_")
    assert ca.status_string(12345) == "unknown status"


def good(**kw):
    base = dict(batch=1, heads=32, kv_heads=8, d=128, n=131072, nq=1, W=256, topk=64, dtype="bf16", chunk=0)
    base.update(kw)
    return ca.params(**base)


def ws_size(p):
    n = ctypes.c_size_t(0)
    rc = ca.load().ca_workspace_size(ctypes.byref(p), ctypes.byref(n))
    return rc, n.value


BAD = [
    (dict(batch=0), ca.CA_ERR_INVALID_ARG, "batch"),
    (dict(heads=0), ca.CA_ERR_INVALID_ARG, "heads"),
    (dict(kv_heads=0), ca.CA_ERR_INVALID_ARG, "heads"),
    (dict(heads=30, kv_heads=8), ca.CA_ERR_INVALID_ARG, "multiple"),
    (dict(n=0), ca.CA_ERR_INVALID_ARG, "n must"),
    (dict(n=2**31), ca.CA_ERR_INVALID_ARG, "n must"),
    (dict(nq=0), ca.CA_ERR_INVALID_ARG, "nq"),
    (dict(n=100, nq=101), ca.CA_ERR_INVALID_ARG, "nq"),
    (dict(W=0), ca.CA_ERR_INVALID_ARG, "W must"),
    (dict(topk=-1), ca.CA_ERR_INVALID_ARG, "topk"),
    (dict(d=96), ca.CA_ERR_UNSUPPORTED, "head dimension"),
    (dict(dtype=7), ca.CA_ERR_UNSUPPORTED, "dtype"),
    (dict(W=4000, topk=96), ca.CA_ERR_UNSUPPORTED, "exceeds"),
    (dict(chunk=300), ca.CA_ERR_INVALID_ARG, "chunk"),
    (dict(chunk=128), ca.CA_ERR_INVALID_ARG, "chunk"),
    (dict(chunk=2048), ca.CA_ERR_INVALID_ARG, "chunk"),
    (dict(topk=513, W=16), ca.CA_ERR_UNSUPPORTED, "topk"),
    # One workgroup per query vector with 32-bit query-vector math: batch * heads * nq < 2^31.
    (dict(batch=2, heads=32, kv_heads=8, n=2**25, nq=2**25, W=64, topk=32), ca.CA_ERR_UNSUPPORTED, "query vectors"),
]


@pytest.mark.parametrize("kw,rc,msg", BAD)
def test_validation_codes(lib, kw, rc, msg):
    p = good(**kw)
    got, _ = ws_size(p)
    assert got == rc
    assert msg in ca.last_error()
    # Every entry point validates the same way before any HIP call.
    vp = ctypes.c_void_p(16)
    assert lib.ca_condensate_attention_ex(ctypes.byref(p), vp, vp, vp, vp, vp, vp, 1 << 40, None) == rc
    assert lib.ca_condensate_select(ctypes.byref(p), vp, vp, vp, vp, 1 << 40, None) == rc
    assert lib.ca_attention_on_subset(ctypes.byref(p), vp, vp, vp, vp, vp, None) == rc


def test_null_params_and_pointers(lib):
    assert lib.ca_workspace_size(None, ctypes.byref(ctypes.c_size_t())) == ca.CA_ERR_INVALID_ARG
    p = good()
    assert lib.ca_workspace_size(ctypes.byref(p), None) == ca.CA_ERR_INVALID_ARG
    vp = ctypes.c_void_p(16)
    assert lib.ca_condensate_attention_ex(ctypes.byref(p), None, vp, vp, vp, vp, vp, 1 << 40, None) == ca.CA_ERR_INVALID_ARG
    assert lib.ca_condensate_select(ctypes.byref(p), vp, None, vp, vp, 1 << 40, None) == ca.CA_ERR_INVALID_ARG
    assert lib.ca_attention_on_subset(ctypes.byref(p), vp, vp, vp, None, vp, None) == ca.CA_ERR_INVALID_ARG
    assert lib.ca_condensate_attention(None, vp, vp, 16, 64, 1, 1, 4, 2, vp, vp) == ca.CA_ERR_INVALID_ARG
    assert lib.ca_condensate_attention(vp, vp, vp, 16, 80, 1, 1, 4, 2, vp, vp) == ca.CA_ERR_UNSUPPORTED


def test_workspace_checks(lib):
    p = good()
    rc, need = ws_size(p)
    assert rc == ca.CA_OK and need > 0
    vp = ctypes.c_void_p(16)
    assert lib.ca_condensate_select(ctypes.byref(p), vp, vp, vp, vp, need - 1, None) == ca.CA_ERR_WORKSPACE
    assert "smaller" in ca.last_error()
    assert lib.ca_condensate_select(ctypes.byref(p), vp, vp, vp, None, need, None) == ca.CA_ERR_WORKSPACE


def test_workspace_size_rules(lib):
    # No candidates (topk = 0, or every position inside the window): no workspace at all.
    assert ws_size(good(topk=0)) == (ca.CA_OK, 0)
    assert ws_size(good(n=200, W=256)) == (ca.CA_OK, 0)
    # Grows with the cache length and with the query count.
    sizes = [ws_size(good(n=n))[1] for n in (4096, 65536, 131072, 1 << 20)]
    assert sizes == sorted(sizes)
    assert ws_size(good(nq=8, n=131072))[1] >= ws_size(good(nq=1, n=131072))[1]
    # Every valid chunk gives a usable plan.
    for c in (0, 256, 512, 1024):
        assert ws_size(good(chunk=c))[0] == ca.CA_OK
    assert ws_size(good(topk=512, W=16))[0] == ca.CA_OK


def test_query_vector_limit(lib):
    # A 1M-token, 32-head prefill at d = 64 takes the matrix-core passes with 2^25 query vectors,
    # more than one grid dimension of 256-wide workgroups holds (2^24): planned, and launched as
    # two-dimensional grids. Up to 2^31 - 1 query vectors are accepted; beyond, nothing runs.
    assert ws_size(good(heads=32, kv_heads=32, d=64, n=2**25, nq=2**25, W=64, topk=32))[0] == ca.CA_OK
    assert ws_size(good(batch=63, heads=32, kv_heads=32, d=64, n=2**20, nq=2**20, W=64, topk=32))[0] == ca.CA_OK
    rc, _ = ws_size(good(batch=64, heads=32, kv_heads=32, d=64, n=2**20, nq=2**20, W=64, topk=32))
    assert rc == ca.CA_ERR_UNSUPPORTED and "query vectors" in ca.last_error()


def test_noscratch_entry_point_rules(lib):
    vp = ctypes.c_void_p(16)
    # Validation first, as every entry point.
    p = good(batch=0)
    assert lib.ca_condensate_attention_noscratch(ctypes.byref(p), vp, vp, vp, vp, vp, None) == ca.CA_ERR_INVALID_ARG
    p = good()
    assert lib.ca_condensate_attention_noscratch(ctypes.byref(p), None, vp, vp, vp, vp, None) == ca.CA_ERR_INVALID_ARG
    # A problem whose workspace exceeds the library's device array: refused before any HIP call.
    big = good(n=1 << 20, batch=4, topk=128)
    rc, need = ws_size(big)
    assert rc == ca.CA_OK and need > 32 * 1024 * 1024
    assert lib.ca_condensate_attention_noscratch(ctypes.byref(big), vp, vp, vp, vp, vp, None) == ca.CA_ERR_UNSUPPORTED
    assert "device array" in ca.last_error()
    # The 131K GQA decode step fits.
    assert ws_size(good())[1] <= 32 * 1024 * 1024


def test_mass_entry_point_rules(lib):
    """The mass diagnostic runs on every scoring path (decode, MFMA prefill, chunked); problems
    without candidate rows, missing pointers and short workspaces are rejected on the host."""
    vp = ctypes.c_void_p(16)
    # A decode (streaming path), a bf16 prefill (MFMA path) and the chunked path: a NULL mass
    # pointer is an argument error, a short workspace a workspace error.
    for p in (ca.Params(batch=1, heads=4, kv_heads=1, d=128, n=4000, nq=1, W=64, topk=32,
                        dtype=ca.CA_BF16, chunk=0),
              ca.Params(batch=1, heads=2, kv_heads=2, d=128, n=2000, nq=600, W=64, topk=64,
                        dtype=ca.CA_BF16, chunk=0),
              ca.Params(batch=1, heads=4, kv_heads=1, d=128, n=4000, nq=1, W=64, topk=32,
                        dtype=ca.CA_BF16, chunk=256)):
        rc, need = ws_size(p)
        assert rc == ca.CA_OK and need > 0
        assert lib.ca_condensate_attention_mass_ex(ctypes.byref(p), vp, vp, vp, vp, vp, None, vp,
                                                   need, None) == ca.CA_ERR_INVALID_ARG
        assert lib.ca_condensate_attention_mass_ex(ctypes.byref(p), vp, vp, vp, vp, vp, vp, vp,
                                                   need - 1, None) == ca.CA_ERR_WORKSPACE
    # No candidate rows (topk = 0; W >= n): unsupported.
    for q in (ca.Params(batch=1, heads=2, kv_heads=2, d=128, n=2000, nq=600, W=64, topk=0,
                        dtype=ca.CA_BF16, chunk=0),
              ca.Params(batch=1, heads=2, kv_heads=2, d=128, n=200, nq=200, W=300, topk=8,
                        dtype=ca.CA_F32, chunk=256)):
        assert lib.ca_condensate_attention_mass_ex(ctypes.byref(q), vp, vp, vp, vp, vp, vp, vp,
                                                   1 << 40, None) == ca.CA_ERR_UNSUPPORTED
        assert "mass diagnostic needs" in ca.last_error()


def test_dense_entry_point_rules(lib):
    vp = ctypes.c_void_p(16)
    p = ca.Params(batch=1, heads=2, kv_heads=2, d=128, n=1000, nq=1000, W=4, topk=2,
                  dtype=ca.CA_F32, chunk=0)
    assert lib.ca_dense_attention_ex(ctypes.byref(p), vp, vp, vp, vp, None) == ca.CA_ERR_UNSUPPORTED
    assert "bfloat16" in ca.last_error()
    p.dtype = ca.CA_BF16
    assert lib.ca_dense_attention_ex(ctypes.byref(p), vp, None, vp, vp, None) == ca.CA_ERR_INVALID_ARG
