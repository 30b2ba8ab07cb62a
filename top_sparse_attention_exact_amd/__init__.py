"""MI355X (gfx950) top-k selection and top-K sparse-attention decode.

Every step runs in the HIP library ``libatopk.so`` (C ABI: ``include/atopk.h``).
The functions here only marshal torch tensors (device memory) and the current
torch stream into that ABI; they allocate outputs and the workspace with torch.
There is no Python or CPU implementation behind them: without the built
library every call raises.

    exact(x, k)                       -> (values, indices)   exact top-k per row
    bucketed(x, k, b, kb, final_exact, assignment=...) -> (values, indices)
                                      two-stage bucketed (interleaved or
                                      contiguous buckets)
    sparse_attn_decode(q, K, V, k_sel, b, kb) -> out (, sel_idx, scores)
    sparse_attn_rerank(q, K, V, cand, window, k_sel) -> out (, sel_idx)
                                      Top-K over a given candidate set
    expected_recall(n, k, b, kb)      finite-n Eq. (1) (host)
    choose(x, k, min_recall)          fastest measured (b, kb) meeting the
                                      recall target, and its result
"""

import ctypes

import torch

from . import _lib
from ._lib import AtopkError, check, lib, status_str  # noqa: F401

F32 = 0
BF16 = 1
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}


def _stream_ptr(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _workspace(nbytes, device):
    if nbytes == 0:
        return None, 0
    # 256-byte alignment: torch's caching allocator hands out 512-byte aligned blocks.
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    assert ws.data_ptr() % 256 == 0
    return ws, nbytes


def _check_rows(x):
    if x.dim() != 2:
        raise ValueError("x must be 2-D [m, n]")
    if x.dtype not in _DTYPES:
        raise TypeError("x must be float32 or bfloat16")
    if x.stride(1) != 1:
        raise ValueError("rows of x must be contiguous (stride(1) == 1)")
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor")


def exact_workspace_bytes(dtype, m, n, k, ldx=None):
    size = ctypes.c_size_t(0)
    check(lib().atopk_exact_workspace(_DTYPES[dtype], m, n, ldx if ldx is not None else n, k, ctypes.byref(size)),
          "atopk_exact_workspace")
    return size.value


INTERLEAVED = 0
CONTIGUOUS = 1
_ASSIGN = {"interleaved": INTERLEAVED, "contiguous": CONTIGUOUS}


def bucketed_workspace_bytes(dtype, m, n, k, b, kb, final_exact, ldx=None, assignment="interleaved"):
    size = ctypes.c_size_t(0)
    check(lib().atopk_bucketed_ex_workspace(_DTYPES[dtype], m, n, ldx if ldx is not None else n, k, b, kb,
                                            int(bool(final_exact)), _ASSIGN[assignment], ctypes.byref(size)),
          "atopk_bucketed_ex_workspace")
    return size.value


def decode_workspace_bytes(batch, hq, hkv, ctx, d, k_sel, b, kb):
    size = ctypes.c_size_t(0)
    check(lib().atopk_sparse_attn_decode_workspace(batch, hq, hkv, ctx, d, k_sel, b, kb, ctypes.byref(size)),
          "atopk_sparse_attn_decode_workspace")
    return size.value


def exact(x, k, workspace=None):
    """Exact top-k of each row of x [m, n]: values (x.dtype) and int32
    indices [m, k], value descending then index ascending."""
    _check_rows(x)
    m, n = x.shape
    ldx = x.stride(0) if m > 1 else n
    vals = torch.empty((m, k), dtype=x.dtype, device=x.device)
    idx = torch.empty((m, k), dtype=torch.int32, device=x.device)
    need = exact_workspace_bytes(x.dtype, m, n, k, ldx)
    ws, nbytes = (workspace, workspace.numel()) if workspace is not None else _workspace(need, x.device)
    st = lib().atopk_exact(_ptr(x), _DTYPES[x.dtype], m, n, ldx, k, _ptr(vals), _ptr(idx), _ptr(ws), nbytes,
                           _stream_ptr(x.device))
    check(st, "atopk_exact")
    return vals, idx


def bucketed(x, k, b, kb, final_exact=True, workspace=None, assignment="interleaved"):
    """Bucketed top-k: exact top-kb in each of b buckets -- interleaved
    (i mod b) or contiguous (floor(i*b/n)) -- then, if final_exact, the exact
    top-k of the b*kb candidates ([m, k], sorted); otherwise the candidates
    themselves, bucket-major [m, b*kb]."""
    _check_rows(x)
    m, n = x.shape
    ldx = x.stride(0) if m > 1 else n
    width = k if final_exact else b * kb
    vals = torch.empty((m, width), dtype=x.dtype, device=x.device)
    idx = torch.empty((m, width), dtype=torch.int32, device=x.device)
    need = bucketed_workspace_bytes(x.dtype, m, n, k, b, kb, final_exact, ldx, assignment)
    ws, nbytes = (workspace, workspace.numel()) if workspace is not None else _workspace(need, x.device)
    if assignment == "interleaved":
        st = lib().atopk_bucketed(_ptr(x), _DTYPES[x.dtype], m, n, ldx, k, b, kb, int(bool(final_exact)),
                                  _ptr(vals), _ptr(idx), _ptr(ws), nbytes, _stream_ptr(x.device))
        check(st, "atopk_bucketed")
    else:
        st = lib().atopk_bucketed_ex(_ptr(x), _DTYPES[x.dtype], m, n, ldx, k, b, kb, int(bool(final_exact)),
                                     _ASSIGN[assignment], _ptr(vals), _ptr(idx), _ptr(ws), nbytes,
                                     _stream_ptr(x.device))
        check(st, "atopk_bucketed_ex")
    return vals, idx


NOALLOC_SCRATCH_BYTES = 32 << 20  # ATOPK_NOALLOC_SCRATCH_BYTES


def bucketed_noalloc(x, k, b, kb, final_exact=True):
    """bucketed() through atopk_bucketed_noalloc: the library's own device
    scratch array is the workspace (no workspace allocation).  Outputs are
    allocated here as usual."""
    _check_rows(x)
    m, n = x.shape
    ldx = x.stride(0) if m > 1 else n
    width = k if final_exact else b * kb
    vals = torch.empty((m, width), dtype=x.dtype, device=x.device)
    idx = torch.empty((m, width), dtype=torch.int32, device=x.device)
    st = lib().atopk_bucketed_noalloc(_ptr(x), _DTYPES[x.dtype], m, n, ldx, k, b, kb, int(bool(final_exact)),
                                      _ptr(vals), _ptr(idx), _stream_ptr(x.device))
    check(st, "atopk_bucketed_noalloc")
    return vals, idx


def sparse_attn_decode(q, K, V, k_sel, b=1, kb=None, scale=None, ctx=None, return_sel=False, return_scores=False,
                       workspace=None):
    """Top-K sparse-attention decode.  q [B, Hq, D], K/V [B, Hkv, Lmax, D]
    bf16 (the first `ctx` keys are live).  (b, kb) = (1, k_sel) is the exact
    Top-K.  Returns out [B, Hq, D] bf16 (plus int32 sel_idx [B, Hq, k_sel]
    and fp32 scores [B, Hq, ctx] when asked)."""
    if kb is None:
        kb = k_sel if b == 1 else None
    for t in (q, K, V):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("q, K, V must be bf16 GPU tensors")
    if not (q.is_contiguous() and K.is_contiguous() and V.is_contiguous()):
        raise ValueError("q, K, V must be contiguous")
    bsz, hq, d = q.shape
    _, hkv, lmax, d2 = K.shape
    if V.shape != K.shape or d2 != d:
        raise ValueError("shape mismatch")
    ctx = lmax if ctx is None else ctx
    scale = (1.0 / d ** 0.5) if scale is None else scale
    out = torch.empty((bsz, hq, d), dtype=torch.bfloat16, device=q.device)
    sel = torch.empty((bsz, hq, k_sel), dtype=torch.int32, device=q.device) if return_sel else None
    scores = torch.empty((bsz, hq, ctx), dtype=torch.float32, device=q.device) if return_scores else None
    need = decode_workspace_bytes(bsz, hq, hkv, ctx, d, k_sel, b, kb)
    ws, nbytes = (workspace, workspace.numel()) if workspace is not None else _workspace(need, q.device)
    st = lib().atopk_sparse_attn_decode(_ptr(q), _ptr(K), _ptr(V), bsz, hq, hkv, ctx, lmax, d, float(scale), k_sel,
                                        b, kb, _ptr(out), _ptr(sel), _ptr(scores), _ptr(ws), nbytes,
                                        _stream_ptr(q.device))
    check(st, "atopk_sparse_attn_decode")
    res = [out]
    if return_sel:
        res.append(sel)
    if return_scores:
        res.append(scores)
    return res[0] if len(res) == 1 else tuple(res)


def sparse_attn_rerank(q, K, V, cand, window, k_sel, scale=None, ctx=None, return_sel=False, return_scores=False,
                       workspace=None):
    """Candidate-set rerank decode.  q [B, Hq, D], K/V [B, Hkv, Lmax, D] bf16;
    cand [B, Hq, C] int32 candidate key indices per query head (entries
    outside [0, ctx) are skipped, repeats count once); the last `window` keys
    are candidates too.  Returns out [B, Hq, D] bf16 (plus int32 sel_idx
    [B, Hq, k_sel], -1 padded, and fp32 scores [B, Hq, ctx] -- NaN except at
    the candidates' positions -- when asked)."""
    for t in (q, K, V):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("q, K, V must be bf16 GPU tensors")
    if not (q.is_contiguous() and K.is_contiguous() and V.is_contiguous()):
        raise ValueError("q, K, V must be contiguous")
    if cand.dtype != torch.int32 or not cand.is_cuda or cand.dim() != 3 or not cand.is_contiguous():
        raise TypeError("cand must be a contiguous int32 GPU tensor [B, Hq, C]")
    bsz, hq, d = q.shape
    _, hkv, lmax, d2 = K.shape
    if V.shape != K.shape or d2 != d or tuple(cand.shape[:2]) != (bsz, hq):
        raise ValueError("shape mismatch")
    ctx = lmax if ctx is None else ctx
    scale = (1.0 / d ** 0.5) if scale is None else scale
    out = torch.empty((bsz, hq, d), dtype=torch.bfloat16, device=q.device)
    sel = torch.empty((bsz, hq, k_sel), dtype=torch.int32, device=q.device) if return_sel else None
    scores = torch.full((bsz, hq, ctx), float("nan"), dtype=torch.float32, device=q.device) if return_scores else None
    ncand = cand.shape[2]
    size = ctypes.c_size_t(0)
    check(lib().atopk_sparse_attn_rerank_workspace(bsz, hq, hkv, ctx, ncand, window, ctypes.byref(size)),
          "atopk_sparse_attn_rerank_workspace")
    ws, nbytes = (workspace, workspace.numel()) if workspace is not None else _workspace(size.value, q.device)
    st = lib().atopk_sparse_attn_rerank(_ptr(q), _ptr(K), _ptr(V), bsz, hq, hkv, ctx, lmax, d, float(scale),
                                        _ptr(cand) if ncand > 0 else ctypes.c_void_p(0), ncand,
                                        ncand, window, k_sel, _ptr(out), _ptr(sel), _ptr(scores), _ptr(ws), nbytes,
                                        _stream_ptr(q.device))
    check(st, "atopk_sparse_attn_rerank")
    res = [out] + ([sel] if return_sel else []) + ([scores] if return_scores else [])
    return res[0] if len(res) == 1 else tuple(res)


_stage_array = None


def stage_events(events):
    """Measurement aid (atopk_stage_events): after this, the calling thread's
    library calls record events[j] on their stream right after enqueuing
    their j-th kernel (counting across calls).  `events` are
    torch.cuda.Event objects created with enable_timing=True and recorded
    once already (so that the HIP event exists); None or [] turns it off.
    Returns nothing; stage_count() gives the marks made so far."""
    global _stage_array
    if not events:
        _stage_array = None
        check(lib().atopk_stage_events(None, 0), "atopk_stage_events")
        return
    arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
    if any(not e.cuda_event for e in events):
        raise ValueError("record each event once before handing it to the library")
    _stage_array = arr
    check(lib().atopk_stage_events(arr, len(events)), "atopk_stage_events")


def stage_count():
    return lib().atopk_stage_count()


def expected_recall(n, k, b, kb):
    """Expected stage-1 recall of (b, kb) on an iid row of n distinct values
    (finite-n form of Eq. (1)); computed by the library on the host."""
    r = ctypes.c_double(0.0)
    check(lib().atopk_expected_recall(n, k, b, kb, ctypes.byref(r)), "atopk_expected_recall")
    return r.value


def choose(x, k, min_recall):
    """Time every (b, kb) whose expected recall reaches min_recall (and the
    exact top-k) on the rows of x and return the fastest:
    dict(b, kb, recall, us, values, indices) -- values / indices [m, k] are
    that configuration's sorted result.  Blocks until the timing finishes."""
    _check_rows(x)
    m, n = x.shape
    ldx = x.stride(0) if m > 1 else n
    size = ctypes.c_size_t(0)
    check(lib().atopk_choose_workspace(_DTYPES[x.dtype], m, n, ldx, k, float(min_recall), ctypes.byref(size)),
          "atopk_choose_workspace")
    ws, nbytes = _workspace(size.value, x.device)
    vals = torch.empty((m, k), dtype=x.dtype, device=x.device)
    idx = torch.empty((m, k), dtype=torch.int32, device=x.device)
    b, kb = ctypes.c_int64(0), ctypes.c_int64(0)
    rec, us = ctypes.c_double(0.0), ctypes.c_float(0.0)
    check(lib().atopk_choose(_ptr(x), _DTYPES[x.dtype], m, n, ldx, k, float(min_recall), _ptr(vals), _ptr(idx),
                             _ptr(ws), nbytes, _stream_ptr(x.device), ctypes.byref(b), ctypes.byref(kb),
                             ctypes.byref(rec), ctypes.byref(us)), "atopk_choose")
    return dict(b=b.value, kb=kb.value, recall=rec.value, us=us.value, values=vals, indices=idx)
