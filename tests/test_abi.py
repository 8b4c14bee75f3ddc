"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/pma.h declares, and rejects bad arguments on the host before any HIP
call (kpnn2 PackedMultiheadAttention page, constructor "Raises")."""
import ctypes
import os
import re

import numpy as np
import pytest

import graph_sparse_head_amd as pma

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pma.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pma_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("pma_create", "pma_forward", "pma_destroy", "pma_nnz", "pma_edges",
              "pma_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(pma.library_path())
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_names_match_header():
    for n in _declared():
        assert hasattr(pma, n), n


def _create_status(src, tgt, nnz=None, L=4, S=4, E=8, H=2, loops=0, dtype=0, plan=True):
    lib = pma._load()
    src = np.ascontiguousarray(src, np.int64)
    tgt = np.ascontiguousarray(tgt, np.int64)
    h = ctypes.c_void_p(1234)
    st = lib.pma_create(ctypes.byref(h) if plan else None,
                        src.ctypes.data if src.size else None,
                        tgt.ctypes.data if tgt.size else None,
                        src.shape[0] if nnz is None else nnz, L, S, E, H, loops, dtype, None)
    if plan:
        assert h.value is None          # *plan is NULL after a failure
    return pma.STATUS[st]


@pytest.mark.parametrize("kw,expect", [
    (dict(src=[], tgt=[]), "PMA_E_INDEX_EMPTY"),
    (dict(src=[0, 4], tgt=[1, 0]), "PMA_E_INDEX_RANGE"),
    (dict(src=[0, -1], tgt=[1, 0]), "PMA_E_INDEX_RANGE"),
    (dict(src=[0, 1], tgt=[1, 4]), "PMA_E_INDEX_RANGE"),
    (dict(src=[0, 4], tgt=[1, 3], L=3, S=5), "PMA_E_INDEX_RANGE"),
    (dict(src=[0], tgt=[0], L=0), "PMA_E_SIZE"),
    (dict(src=[0], tgt=[0], S=0), "PMA_E_SIZE"),
    (dict(src=[0], tgt=[0], E=0), "PMA_E_SIZE"),
    (dict(src=[0], tgt=[0], H=0), "PMA_E_SIZE"),
    (dict(src=[0], tgt=[0], E=6, H=4), "PMA_E_SIZE"),
    (dict(src=[0], tgt=[0], L=3, S=4, loops=1), "PMA_E_SELF_LOOPS"),
    (dict(src=[0], tgt=[0], loops=2), "PMA_E_ARG"),
    (dict(src=[0], tgt=[0], dtype=5), "PMA_E_DTYPE"),
    (dict(src=[0], tgt=[0], plan=False), "PMA_E_NULL"),
])
def test_create_rejects(kw, expect):
    assert _create_status(**kw) == expect
    assert pma.pma_last_error() != ""


def test_create_null_indices():
    lib = pma._load()
    h = ctypes.c_void_p()
    st = lib.pma_create(ctypes.byref(h), None, None, 3, 4, 4, 8, 2, 0, 0, None)
    assert pma.STATUS[st] == "PMA_E_NULL"


def test_binding_rejects_before_the_library():
    with pytest.raises(pma.PmaError) as e:
        pma.pma_create([0, 1], [1], 2, 2, 4, 2)
    assert e.value.name == "PMA_E_ARG"
    with pytest.raises(pma.PmaError) as e:
        pma.pma_create([0.5], [1], 2, 2, 4, 2)
    assert e.value.name == "PMA_E_ARG"
    with pytest.raises(pma.PmaError) as e:
        pma.pma_create([0], [1], 2, 2, 4, 2, dtype="f16")
    assert e.value.name == "PMA_E_DTYPE"
    with pytest.raises(pma.PmaError) as e:
        pma.pma_create([0], [1], 2, 2, 4, 2, add_self_loops=1)
    assert e.value.name == "PMA_E_ARG"
    with pytest.raises(pma.PmaError) as e:
        pma.pma_create([], [], 2, 2, 4, 2)
    assert e.value.name == "PMA_E_INDEX_EMPTY"


def test_null_plan_calls():
    lib = pma._load()
    assert lib.pma_destroy(None) == 0
    assert lib.pma_nnz(None) == -1
    z = ctypes.c_void_p(0x10)
    st = lib.pma_forward(None, 1, z, z, z, z, None, z, None, z, None, z, None, z, None, 0, None)
    assert pma.STATUS[st] == "PMA_E_NULL"
    ms = np.zeros(5)
    calls = np.zeros(5, np.int64)
    assert pma.STATUS[lib.pma_profile_read(None, ms.ctypes.data, calls.ctypes.data)] == "PMA_E_NULL"
    assert pma.STATUS[lib.pma_edges(None, None, None)] == "PMA_E_NULL"
    assert pma.STATUS[lib.pma_profile_stages(None, 1)] == "PMA_E_NULL"


def test_create_graph_rejects():
    lib = pma._load()
    src = np.array([0, 1], np.int64)
    tgt = np.array([1, 1], np.int64)
    for args, expect in (((0, 2, 2), "PMA_E_INDEX_EMPTY"), ((2, 0, 2), "PMA_E_SIZE"),
                         ((2, 2, 0), "PMA_E_SIZE")):
        h = ctypes.c_void_p(1234)
        n, L, S = args
        st = lib.pma_create_graph(ctypes.byref(h), src.ctypes.data, tgt.ctypes.data, n, L, S, 0,
                                  0, None)
        assert pma.STATUS[st] == expect and h.value is None
    h = ctypes.c_void_p(1234)
    st = lib.pma_create_graph(ctypes.byref(h), src.ctypes.data, tgt.ctypes.data, 2, 2, 3, 1, 0,
                              None)
    assert pma.STATUS[st] == "PMA_E_SELF_LOOPS" and h.value is None
    with pytest.raises(pma.PmaError) as e:
        pma.pma_create_graph([0, 1], [1], 2, 2)
    assert e.value.name == "PMA_E_ARG"


def test_null_plan_linear_calls():
    lib = pma._load()
    z = ctypes.c_void_p(0x10)
    assert pma.STATUS[lib.pma_linear_forward(None, 1, 1, z, z, None, z, None)] == "PMA_E_NULL"
    assert pma.STATUS[lib.pma_linear_backward(None, 1, 1, z, z, z, z, z, None, None)] == \
        "PMA_E_NULL"


# ---------------------------------------------------------------------------
# pma_edge_list: the library's host-side index rules against the oracle's


@pytest.mark.parametrize("seed", range(30))
def test_edge_list_matches_oracle(seed):
    import oracle
    from graph_sparse_head_amd import synth
    rng = np.random.default_rng(300 + seed)
    L = int(rng.integers(1, 40))
    S = L if rng.random() < 0.5 else int(rng.integers(1, 40))
    src, tgt = synth.random_graph(rng, L, S, float(rng.uniform(0.05, 0.5)))
    if src.size == 0:
        src, tgt = np.array([0]), np.array([0])
    perm = rng.permutation(src.size)
    src, tgt = src[perm], tgt[perm]
    loops = L == S and bool(rng.random() < 0.6)
    s, t = pma.pma_edge_list(src, tgt, L, S, add_self_loops=loops)
    rs, rt = oracle.prepare_edges(src, tgt, L, S, 1, 1, loops)
    assert (s == rs).all() and (t == rt).all()


@pytest.mark.parametrize("kw,expect", [
    (dict(src=[], tgt=[]), "PMA_E_INDEX_EMPTY"),
    (dict(src=[0, 4], tgt=[1, 0]), "PMA_E_INDEX_RANGE"),
    (dict(src=[0, 1], tgt=[1, -1]), "PMA_E_INDEX_RANGE"),
    (dict(src=[0, 1, 0], tgt=[1, 2, 1]), "PMA_E_INDEX_DUPLICATE"),
    (dict(src=[0, 1], tgt=[1, 2], L=3, S=5, loops=True), "PMA_E_SELF_LOOPS"),
    (dict(src=[0], tgt=[0], L=0), "PMA_E_SIZE"),
])
def test_edge_list_rejects(kw, expect):
    L, S = kw.get("L", 4), kw.get("S", 4)
    with pytest.raises(pma.PmaError) as e:
        pma.pma_edge_list(np.array(kw["src"], np.int64), np.array(kw["tgt"], np.int64), L, S,
                          add_self_loops=kw.get("loops", False))
    assert e.value.name == expect


def test_edge_list_reports_its_length_when_capacity_is_short():
    lib = pma._load()
    src = np.array([0, 1], np.int64)
    tgt = np.array([1, 0], np.int64)
    out = np.empty(8, np.int64)
    n = ctypes.c_int64(-1)
    st = lib.pma_edge_list(src.ctypes.data, tgt.ctypes.data, 2, 3, 3, 1, 2, out.ctypes.data,
                           out.ctypes.data, ctypes.byref(n))
    assert pma.STATUS[st] == "PMA_E_SIZE" and n.value == 5


def test_gather_ceiling_rejects_before_any_launch():
    # argument checks of the calibration entry point (no device memory is
    # touched: every call below returns before a launch)
    lib = pma._load()
    z = ctypes.c_void_p(0x1000)
    st = lambda *a: pma.STATUS[lib.pma_gather_ceiling(*a)]
    assert st(None, 1024, z, 8, 8, z, None) == "PMA_E_NULL"
    assert st(z, 1024, None, 8, 8, z, None) == "PMA_E_NULL"
    assert st(z, 1024, z, 8, 8, None, None) == "PMA_E_NULL"
    for tb in (0, 1000, 1536, 1 << 32):
        assert st(z, tb, z, 8, 8, z, None) == "PMA_E_ARG", tb
    for n, per in ((0, 8), (8, 0), (8, (1 << 20) + 1), (-1, 8), ((1 << 31) + 1, 1)):
        assert st(z, 1024, z, n, per, z, None) == "PMA_E_ARG", (n, per)
    assert "rows_per_wave" in pma.pma_last_error() or "wavefronts" in pma.pma_last_error()
