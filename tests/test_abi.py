"""The C ABI boundary on the CPU: the library loads, exports every entry
point include/atopk.h declares, and every argument error is reported before
any HIP call (so these run without a GPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "atopk.h")

lib_mod = pytest.importorskip("top_sparse_attention_exact_amd._lib")

if not os.path.exists(lib_mod.LIB_PATH):
    pytest.skip("libatopk.so not built", allow_module_level=True)

OK, ENULL, ESHAPE, EPARAM, EUNSUP, EWS, EHIP = range(7)
F32, BF16 = 0, 1


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(atopk_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return lib_mod.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) == 18
    handle = ctypes.CDLL(lib_mod.LIB_PATH)
    for name in names:
        assert hasattr(handle, name), name
    assert set(names) == set(lib_mod.EXPORTED)


def test_status_strings(L):
    for s in range(7):
        assert L.atopk_status_str(s)
    assert L.atopk_status_str(99) == b"unknown status"
    assert L.atopk_version() >= 100


def test_stage_events_arguments(L):
    """The measurement hook validates its arguments, counts marks only from
    entry points that launch, and turns off with count 0 (no HIP call)."""
    assert L.atopk_stage_events(None, -1) == EPARAM
    assert L.atopk_stage_events(None, 3) == EPARAM
    assert L.atopk_stage_events(None, 0) == OK
    assert L.atopk_stage_count() == 0
    # a call that fails validation launches nothing, so marks nothing
    sz = ctypes.c_size_t(0)
    assert L.atopk_exact(None, F32, 1, 10, 10, 5, None, None, None, 0, None) == ENULL
    assert L.atopk_stage_count() == 0


def test_noalloc_validation(L):
    """The no-allocation variant refuses, before any HIP call, what
    atopk_bucketed refuses, and shapes whose workspace exceeds its array."""
    big = ctypes.c_size_t(0)
    assert L.atopk_bucketed_workspace(F32, 8, 1 << 24, 1 << 24, 64, 4096, 16, 1, ctypes.byref(big)) == OK
    assert big.value > 32 << 20
    assert L.atopk_bucketed_noalloc(FAKE, F32, 8, 1 << 24, 1 << 24, 64, 4096, 16, 1, FAKE, FAKE, None) == EWS
    assert L.atopk_bucketed_noalloc(FAKE, F32, 2, 100, 99, 5, 4, 2, 1, FAKE, FAKE, None) == ESHAPE  # ldx < n
    assert L.atopk_bucketed_noalloc(FAKE, F32, 2, 100, 100, 50, 4, 2, 1, FAKE, FAKE, None) == EPARAM  # b*kb < k
    assert L.atopk_bucketed_noalloc(FAKE, 7, 2, 100, 100, 5, 4, 2, 1, FAKE, FAKE, None) == EUNSUP  # dtype
    assert L.atopk_bucketed_noalloc(None, F32, 0, 100, 100, 5, 4, 2, 1, None, None, None) == OK  # m == 0


def _ws_exact(L, dt, m, n, ldx, k):
    sz = ctypes.c_size_t(0)
    return L.atopk_exact_workspace(dt, m, n, ldx, k, ctypes.byref(sz)), sz.value


def _ws_bucketed(L, dt, m, n, ldx, k, b, kb, fin):
    sz = ctypes.c_size_t(0)
    return L.atopk_bucketed_workspace(dt, m, n, ldx, k, b, kb, fin, ctypes.byref(sz)), sz.value


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails validation first


def test_exact_validation(L):
    assert _ws_exact(L, F32, 4, 100, 100, 10)[0] == OK
    assert _ws_exact(L, F32, -1, 100, 100, 10)[0] == ESHAPE
    assert _ws_exact(L, F32, 4, 0, 100, 1)[0] == ESHAPE
    assert _ws_exact(L, F32, 4, 100, 99, 10)[0] == ESHAPE  # ldx < n
    assert _ws_exact(L, F32, 4, 100, 100, 0)[0] == ESHAPE
    assert _ws_exact(L, F32, 4, 100, 100, 101)[0] == ESHAPE  # k > n
    assert _ws_exact(L, 7, 4, 100, 100, 10)[0] == EUNSUP
    assert _ws_exact(L, F32, 4, 20000, 20000, 8193)[0] == EUNSUP  # k > 8192
    assert _ws_exact(L, F32, 1, 1 << 31, 1 << 31, 10)[0] == EUNSUP
    assert L.atopk_exact_workspace(F32, 4, 100, 100, 10, None) == ENULL
    # null pointers
    assert L.atopk_exact(None, F32, 4, 100, 100, 10, FAKE, FAKE, None, 0, None) == ENULL
    assert L.atopk_exact(FAKE, F32, 4, 100, 100, 10, None, FAKE, None, 0, None) == ENULL
    assert L.atopk_exact(FAKE, F32, 4, 100, 100, 10, FAKE, None, None, 0, None) == ENULL
    # m == 0 is a no-op, even with null pointers
    assert L.atopk_exact(None, F32, 0, 100, 100, 10, None, None, None, 0, None) == OK
    # elements and indices must be aligned to their size
    odd2, odd1 = ctypes.c_void_p(0x1002), ctypes.c_void_p(0x1001)
    assert L.atopk_exact(odd2, F32, 4, 100, 100, 10, FAKE, FAKE, None, 0, None) == EPARAM
    assert L.atopk_exact(FAKE, F32, 4, 100, 100, 10, odd2, FAKE, None, 0, None) == EPARAM
    assert L.atopk_exact(FAKE, BF16, 4, 100, 100, 10, FAKE, odd2, None, 0, None) == EPARAM
    assert L.atopk_exact(odd1, BF16, 4, 100, 100, 10, FAKE, FAKE, None, 0, None) == EPARAM
    assert L.atopk_bucketed(odd2, F32, 2, 100, 100, 4, 4, 1, 1, FAKE, FAKE, None, 0, None) == EPARAM
    assert L.atopk_bucketed_ex(odd1, BF16, 2, 100, 100, 4, 4, 1, 1, 0, FAKE, FAKE, None, 0, None) == EPARAM


def test_exact_workspace_checks(L):
    st, need = _ws_exact(L, F32, 64, 1 << 20, 1 << 20, 8192)  # split rows need a workspace
    assert st == OK and need > 0
    assert L.atopk_exact(FAKE, F32, 64, 1 << 20, 1 << 20, 8192, FAKE, FAKE, None, 0, None) == EWS
    assert L.atopk_exact(FAKE, F32, 64, 1 << 20, 1 << 20, 8192, FAKE, FAKE, FAKE, need - 1, None) == EWS
    assert L.atopk_exact(FAKE, F32, 64, 1 << 20, 1 << 20, 8192, FAKE, FAKE, ctypes.c_void_p(0x1008), need, None) == EWS


def test_bucketed_validation(L):
    assert _ws_bucketed(L, BF16, 256, 131072, 131072, 64, 128, 2, 1)[0] == OK
    assert _ws_bucketed(L, BF16, 256, 131072, 131072, 64, 0, 2, 1)[0] == EPARAM
    assert _ws_bucketed(L, BF16, 256, 131072, 131072, 64, 64, 0, 1)[0] == EPARAM
    assert _ws_bucketed(L, BF16, 256, 131072, 131072, 64, 31, 2, 1)[0] == EPARAM  # b*kb < k
    assert _ws_bucketed(L, BF16, 256, 131072, 131072, 64, 31, 2, 0)[0] == EPARAM
    assert _ws_bucketed(L, F32, 1, 100, 100, 4, 30, 4, 1)[0] == EPARAM  # kb > floor(n/b)
    assert _ws_bucketed(L, F32, 1, 100, 100, 4, 101, 1, 1)[0] == EPARAM  # b > n
    assert _ws_bucketed(L, F32, 1, 10000, 10000, 64, 8, 17, 1)[0] == EUNSUP  # kb > 16
    assert _ws_bucketed(L, F32, 1, 10000, 10000, 64, 1, 64, 1)[0] == OK  # exact route
    assert _ws_bucketed(L, F32, 1, 10000, 10000, 10, 1, 20, 1)[0] == EUNSUP  # b = 1 but kb != k, kb > 16
    assert _ws_bucketed(L, F32, 1, 20000, 20000, 8193, 1024, 16, 1)[0] == EUNSUP
    assert _ws_bucketed(L, F32, 1, 100, 99, 4, 4, 1, 1)[0] == ESHAPE
    assert L.atopk_bucketed(None, F32, 2, 100, 100, 4, 4, 1, 1, FAKE, FAKE, None, 0, None) == ENULL
    assert L.atopk_bucketed(None, F32, 0, 100, 100, 4, 4, 1, 1, None, None, None, 0, None) == OK
    st, need = _ws_bucketed(L, BF16, 256, 131072, 131072, 64, 128, 2, 1)
    assert st == OK and need > 0
    assert L.atopk_bucketed(FAKE, BF16, 256, 131072, 131072, 64, 128, 2, 1, FAKE, FAKE, None, 0, None) == EWS


def _ws_bucketed_ex(L, dt, m, n, ldx, k, b, kb, fin, assign):
    sz = ctypes.c_size_t(0)
    return L.atopk_bucketed_ex_workspace(dt, m, n, ldx, k, b, kb, fin, assign, ctypes.byref(sz)), sz.value


def test_bucketed_ex_validation(L):
    INTER, CONTIG = 0, 1
    # interleaved: same answers and workspace as atopk_bucketed
    st, need = _ws_bucketed_ex(L, BF16, 256, 131072, 131072, 64, 128, 2, 1, INTER)
    assert (st, need) == _ws_bucketed(L, BF16, 256, 131072, 131072, 64, 128, 2, 1)
    # contiguous: no workspace
    assert _ws_bucketed_ex(L, BF16, 256, 131072, 131072, 64, 128, 2, 1, CONTIG) == (OK, 0)
    assert _ws_bucketed_ex(L, F32, 3, 1000, 1000, 64, 7, 16, 0, CONTIG) == (OK, 0)
    assert _ws_bucketed_ex(L, F32, 3, 1000, 1000, 64, 8, 2, 1, 2)[0] == EPARAM  # unknown assignment
    assert _ws_bucketed_ex(L, F32, 3, 1000, 1000, 64, 8, 2, 1, -1)[0] == EPARAM
    assert _ws_bucketed_ex(L, F32, 3, 1000, 1000, 64, 31, 2, 1, CONTIG)[0] == EPARAM  # b*kb < k
    assert _ws_bucketed_ex(L, F32, 1, 20000, 20000, 64, 1024, 16, 1, CONTIG)[0] == EUNSUP  # 16384 candidates
    assert _ws_bucketed_ex(L, F32, 1, 20000, 20000, 64, 1024, 16, 0, CONTIG)[0] == OK  # no final stage
    assert L.atopk_bucketed_ex_workspace(F32, 1, 100, 100, 4, 4, 1, 1, CONTIG, None) == ENULL
    assert L.atopk_bucketed_ex(None, F32, 2, 100, 100, 4, 4, 1, 1, CONTIG, FAKE, FAKE, None, 0, None) == ENULL
    assert L.atopk_bucketed_ex(None, F32, 0, 100, 100, 4, 4, 1, 1, CONTIG, None, None, None, 0, None) == OK
    assert L.atopk_bucketed_ex(FAKE, F32, 2, 100, 100, 4, 4, 1, 1, 5, FAKE, FAKE, None, 0, None) == EPARAM


def _ws_decode(L, bsz, hq, hkv, ctx, d, ks, b, kb):
    sz = ctypes.c_size_t(0)
    return L.atopk_sparse_attn_decode_workspace(bsz, hq, hkv, ctx, d, ks, b, kb, ctypes.byref(sz)), sz.value


def test_decode_validation(L):
    assert _ws_decode(L, 16, 32, 32, 32768, 128, 512, 256, 2)[0] == OK
    assert _ws_decode(L, 4, 32, 8, 131072, 128, 512, 512, 4)[0] == OK
    assert _ws_decode(L, 4, 32, 8, 131072, 128, 512, 1, 512)[0] == OK  # exact Top-K
    assert _ws_decode(L, 4, 30, 8, 1024, 128, 16, 16, 1)[0] == ESHAPE  # hq % hkv
    assert _ws_decode(L, 4, 32, 8, 1024, 128, 2000, 1, 2000)[0] == ESHAPE  # k_sel > ctx
    assert _ws_decode(L, 4, 32, 8, 1024, 64, 16, 16, 1)[0] == EUNSUP  # d != 128
    assert _ws_decode(L, 4, 32, 2, 1024, 128, 16, 16, 1)[0] == EUNSUP  # group of 16 heads
    assert _ws_decode(L, 4, 32, 8, 1024, 128, 16, 8, 1)[0] == EPARAM  # b*kb < k_sel
    assert _ws_decode(L, 4, 32, 8, 1024, 128, 16, 512, 4)[0] == EPARAM  # kb > ctx/b
    f = ctypes.c_float(0.1)
    assert L.atopk_sparse_attn_decode(None, FAKE, FAKE, 1, 8, 8, 256, 256, 128, f, 16, 16, 1, FAKE, None, None, None,
                                      0, None) == ENULL
    assert L.atopk_sparse_attn_decode(FAKE, FAKE, FAKE, 1, 8, 8, 256, 255, 128, f, 16, 16, 1, FAKE, None, None, None,
                                      0, None) == ESHAPE  # ctx_stride < ctx
    assert L.atopk_sparse_attn_decode(ctypes.c_void_p(0x1004), FAKE, FAKE, 1, 8, 8, 256, 256, 128, f, 16, 16, 1, FAKE,
                                      None, None, None, 0, None) == EUNSUP  # misaligned q
    assert L.atopk_sparse_attn_decode(FAKE, FAKE, FAKE, 1, 8, 8, 256, 256, 128, f, 16, 16, 1, FAKE, None, None, None,
                                      0, None) == EWS


def test_rerank_validation(L):
    def call(bsz=2, hq=8, hkv=2, ctx=4096, stride=4096, d=128, cand=FAKE, ncand=100, cstride=128, window=64,
             k=64, q=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return L.atopk_sparse_attn_rerank(q, FAKE, FAKE, bsz, hq, hkv, ctx, stride, d, 0.1, cand, ncand, cstride,
                                          window, k, out, None, None, ws, ws_bytes, None)
    assert call(hq=6, hkv=4) == ESHAPE          # hq % hkv
    assert call(stride=100) == ESHAPE           # ctx_stride < ctx
    assert call(cstride=50) == ESHAPE           # cand_stride < ncand
    assert call(ncand=-1) == ESHAPE
    assert call(k=0) == ESHAPE
    assert call(window=0) == EPARAM
    assert call(window=5000) == EPARAM          # window > ctx
    assert call(d=64) == EUNSUP
    assert call(ctx=300000, stride=300000) == EUNSUP
    assert call(ncand=8150, cstride=8192) == EUNSUP  # ncand + window > 8192
    assert call(k=8193) == EUNSUP
    assert call(bsz=0, q=None, out=None, cand=None) == OK
    assert call(q=None) == ENULL
    assert call(cand=None) == ENULL
    assert call(q=ctypes.c_void_p(0x1008)) == EUNSUP  # misaligned
    sz = ctypes.c_size_t(0)
    assert L.atopk_sparse_attn_rerank_workspace(2, 8, 2, 4096, 100, 64, None) == ENULL
    assert L.atopk_sparse_attn_rerank_workspace(2, 8, 2, 4096, 100, 0, ctypes.byref(sz)) == EPARAM
    assert L.atopk_sparse_attn_rerank_workspace(2, 8, 2, 4096, 8150, 64, ctypes.byref(sz)) == EUNSUP
    assert L.atopk_sparse_attn_rerank_workspace(2, 8, 2, 4096, 100, 64, ctypes.byref(sz)) == OK
    assert sz.value >= 2 * 8 * (100 + 64) * 8
    assert call(ws=None, ws_bytes=0) == EWS
    assert call(ws_bytes=sz.value - 1) == EWS
    assert call(ws=ctypes.c_void_p(0x1008)) == EWS  # not 256-byte aligned


@pytest.mark.parametrize("n,k,b,kb", [(131072, 64, 64, 1), (131072, 64, 128, 2), (4096, 64, 32, 2), (37, 8, 5, 2),
                                      (128256, 256, 1024, 1), (128256, 256, 512, 2), (2653751, 100, 2048, 1),
                                      (2653751, 100, 64, 2), (1 << 20, 8192, 512, 16), (100, 100, 1, 100),
                                      (1000, 10, 1000, 1)])
def test_expected_recall_matches_oracle(L, n, k, b, kb):
    """The library's host recall model against the oracle's finite-n Eq.(1)
    (itself pinned by exhaustive enumeration)."""
    import oracle

    r = ctypes.c_double(0.0)
    assert L.atopk_expected_recall(n, k, b, kb, ctypes.byref(r)) == OK
    assert r.value == pytest.approx(oracle.eq1_finite(n, k, b, kb), rel=1e-7, abs=1e-9)


def test_expected_recall_and_choose_validation(L):
    r = ctypes.c_double(0.0)
    assert L.atopk_expected_recall(100, 10, 4, 1, None) == ENULL
    assert L.atopk_expected_recall(100, 0, 4, 1, ctypes.byref(r)) == ESHAPE
    assert L.atopk_expected_recall(100, 101, 4, 1, ctypes.byref(r)) == ESHAPE
    assert L.atopk_expected_recall(100, 10, 4, 2, ctypes.byref(r)) == EPARAM  # b*kb < k
    assert L.atopk_expected_recall(100, 10, 101, 1, ctypes.byref(r)) == EPARAM
    assert L.atopk_expected_recall(100, 10, 10, 11, ctypes.byref(r)) == EPARAM  # kb > n/b
    sz = ctypes.c_size_t(0)
    assert L.atopk_choose_workspace(F32, 64, 128256, 128256, 256, 0.9, None) == ENULL
    assert L.atopk_choose_workspace(F32, 64, 128256, 128256, 256, 1.5, ctypes.byref(sz)) == EPARAM
    assert L.atopk_choose_workspace(F32, 64, 128256, 128256, 256, float("nan"), ctypes.byref(sz)) == EPARAM
    assert L.atopk_choose_workspace(F32, 64, 128256, 128256, 0, 0.9, ctypes.byref(sz)) == ESHAPE
    assert L.atopk_choose_workspace(F32, 64, 128256, 128256, 256, 0.9, ctypes.byref(sz)) == OK
    assert sz.value > 0
    b, kb = ctypes.c_int64(0), ctypes.c_int64(0)
    assert L.atopk_choose(None, F32, 64, 128256, 128256, 256, 0.9, FAKE, FAKE, FAKE, sz.value, None,
                          ctypes.byref(b), ctypes.byref(kb), None, None) == ENULL
    assert L.atopk_choose(FAKE, F32, 64, 128256, 128256, 256, 0.9, FAKE, FAKE, None, 0, None,
                          ctypes.byref(b), ctypes.byref(kb), None, None) == EWS
    assert L.atopk_choose(FAKE, F32, 64, 128256, 128256, 256, 0.9, FAKE, FAKE, FAKE, sz.value, None,
                          None, ctypes.byref(kb), None, None) == ENULL
    assert L.atopk_choose(None, F32, 0, 128256, 128256, 256, 0.9, None, None, None, 0, None,
                          ctypes.byref(b), ctypes.byref(kb), None, None) == OK
    assert (b.value, kb.value) == (1, 256)
