"""Exact and bucketed top-k, written from their definitions (CPU, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Readings taken where the pages are silent:

* Ties: the total order is value descending, then the LOWER index first, in
  every stage (the pages do not say how ties break; this makes every result
  unique, so results can be compared exactly).
* -0.0 and +0.0 are equal values (IEEE); their tie is broken by index.  The
  returned value is the element's own bit pattern.
* NaN is outside the domain: inputs are asserted NaN-free.
* bf16 inputs arrive as their raw uint16 bit patterns and are widened
  exactly (bf16 -> fp32 -> fp64 is exact).
"""

import numpy as np


def to_f64(x, dtype):
    """Exact float64 image of an fp32 array or of bf16 bit patterns (uint16).

    Adding +0.0 turns -0.0 into +0.0 so that the two zeros compare equal in
    every later step and ties between them fall to the index rule.
    """
    x = np.asarray(x)
    if dtype == "f32":
        assert x.dtype == np.float32, x.dtype
        v = x.astype(np.float64)
    elif dtype == "bf16":
        assert x.dtype == np.uint16, x.dtype
        v = (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    elif dtype == "f64":
        v = x.astype(np.float64)
    else:
        raise ValueError(dtype)
    assert not np.isnan(v).any(), "NaN inputs are outside the method's domain"
    return v + 0.0


def _rank_order(vals, idx):
    """Positions of (vals, idx) sorted by value desc, then index asc."""
    # np.lexsort sorts by the LAST key first.
    return np.lexsort((idx, -vals))


def exact_topk(x, k, dtype="f32"):
    """Exact top-k of every row of x (shape [m, n]).

    Each row's k greatest values with their positions (the exact problem of
    the Approximate Top-k page, "The reading"), ordered by value descending
    and then by index ascending.

    Returns (idx [m, k] int64, vals [m, k] in x's own dtype / bit pattern).
    """
    x = np.asarray(x)
    assert x.ndim == 2
    m, n = x.shape
    assert 1 <= k <= n
    v = to_f64(x, dtype)
    idx = np.empty((m, k), dtype=np.int64)
    positions = np.arange(n, dtype=np.int64)
    for r in range(m):
        order = _rank_order(v[r], positions)
        idx[r] = order[:k]
    vals = np.take_along_axis(x, idx, axis=1)
    return idx, vals


def bucket_members(n, b, r):
    """Indices of interleaved bucket r: r, r + b, r + 2b, ... < n.

    Interleaved buckets (Approximate Top-k page, "What carries the argument";
    "What would settle it" identifies a bucket with one residue class modulo
    b).  When b does not divide n the first n mod b buckets hold one element
    more (Figure 2: n = 11, b = 3 gives sizes 4, 4, 3).
    """
    return np.arange(r, n, b, dtype=np.int64)


def contiguous_members(n, b, r):
    """Indices of contiguous bucket r: the i with floor(i * b / n) == r.

    The contiguous assignment the Approximate Top-k page compares against the
    interleaved one (Figure 6: recall on correlated inputs; Figure 8:
    runtime).  The page gives no formula; the plainest reading is b blocks of
    consecutive positions, bucket(i) = floor(i * b / n), whose sizes differ by
    at most one when b does not divide n.
    """
    i = np.arange(n, dtype=np.int64)
    return i[(i * b) // n == r]


def bucketed_topk(x, k, b, kb, final_exact, dtype="f32", assignment="interleaved"):
    """Two-stage bucketed top-k (Approximate Top-k page, "What carries the
    argument"): position i belongs to bucket i mod b; stage 1 keeps the k_b
    best of every bucket on its own; stage 2, when asked for, is the exact
    top-k over the b * k_b stage-1 survivors.  assignment="contiguous" uses
    the contiguous buckets of contiguous_members instead.

    Stage 1 output (final_exact False): [m, b * kb], bucket-major, slot
    r * kb + j holding the j-th best element of bucket r.
    Final output (final_exact True): [m, k] sorted by value desc, index asc
    (the index is the element's position in the original row).

    Returns (idx, vals) like exact_topk.
    """
    x = np.asarray(x)
    assert x.ndim == 2
    m, n = x.shape
    assert 1 <= b <= n and 1 <= kb
    assert kb <= n // b, "every bucket must hold at least k_b elements"
    assert b * kb >= k >= 1, "the invariant b * k_b >= k"
    v = to_f64(x, dtype)
    members_of = {"interleaved": bucket_members, "contiguous": contiguous_members}[assignment]
    cand = np.empty((m, b * kb), dtype=np.int64)
    for r in range(b):
        members = members_of(n, b, r)
        for row in range(m):
            order = _rank_order(v[row, members], members)
            cand[row, r * kb:(r + 1) * kb] = members[order[:kb]]
    if not final_exact:
        return cand, np.take_along_axis(x, cand, axis=1)
    idx = np.empty((m, k), dtype=np.int64)
    for row in range(m):
        cv = v[row, cand[row]]
        order = _rank_order(cv, cand[row])
        idx[row] = cand[row, order[:k]]
    return idx, np.take_along_axis(x, idx, axis=1)
