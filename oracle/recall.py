"""Recall of a top-k result and the pages' recall models (CPU, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Approximate Top-k for Increased Parallelism" (Pith review page),
"What carries the argument": Eq. (1) is the expected recall
E[R(k, b, k_b)] = (1/k) (k_b + sum_{i=k_b}^{k-1} F(k_b - 1; i, 1/b)) under
the assumption that the top values fall uniformly over the buckets; Eq. (2)
is the worst case, when all top values sit in ceil(b k / n) buckets.

Readings (the pages leave these open):

* F(x; i, p) is the binomial CDF P(Bin(i, p) <= x).
* Eq. (2) is not printed; only its description is.  With s = n / b elements
  per bucket (b divides n) and k_b <= s, filling as few buckets as possible
  (s top values per bucket) gives recall (k_b floor(k/s) + min(k_b, k mod s))/k.
* Finite n: Eq. (1) draws bucket labels with replacement.  For an iid row of
  distinct values with b dividing n, the exact expectation replaces the
  binomial by a hypergeometric: the i-th largest value survives stage 1 iff
  fewer than k_b of the i larger values share its bucket, and those i values
  are a uniform i-subset of the other n - 1 positions, s - 1 of which are in
  its bucket.  When b does not divide n, buckets i mod b hold ceil(n/b)
  (the first n mod b of them) or floor(n/b) elements; the i-th largest value
  sits at a uniform position, so its bucket has each size with probability
  proportional to the elements of that size, and the hypergeometric term is
  averaged over the two sizes.
"""

import math

import numpy as np


def recall(out_idx, exact_idx):
    """Per-row index recall |S_out & S_exact| / k, k = len(exact row)."""
    out_idx = np.atleast_2d(out_idx)
    exact_idx = np.atleast_2d(exact_idx)
    k = exact_idx.shape[1]
    return np.array([len(np.intersect1d(o, e)) / k for o, e in zip(out_idx, exact_idx)])


def recall_by_bucket_counts(exact_idx, n, b, kb, assignment="interleaved"):
    """Recall computed without running the method: with t_r the number of
    true top-k indices in bucket r, stage 1 keeps min(k_b, t_r) of them, so
    R = sum_r min(k_b, t_r) / k.  Used as an identity check of the oracle.
    Buckets: i mod b (interleaved) or floor(i * b / n) (contiguous)."""
    exact_idx = np.atleast_2d(exact_idx)
    k = exact_idx.shape[1]
    out = []
    for row in exact_idx:
        row = np.asarray(row, dtype=np.int64)
        bucket = row % b if assignment == "interleaved" else (row * b) // n
        t = np.bincount(bucket, minlength=b)
        out.append(np.minimum(t, kb).sum() / k)
    return np.array(out)


def value_recall(out_vals_f64, exact_vals_f64):
    """Secondary recall for tie-heavy data: the share of the k slots whose
    value reaches the exact k-th value, min(k, #{out >= v_k}) / k."""
    out_vals_f64 = np.atleast_2d(out_vals_f64)
    exact_vals_f64 = np.atleast_2d(exact_vals_f64)
    k = exact_vals_f64.shape[1]
    kth = exact_vals_f64[:, -1:]
    return np.minimum(k, (out_vals_f64 >= kth).sum(axis=1)) / k


def binom_cdf(x, i, p):
    """P(Bin(i, p) <= x), summed term by term."""
    if x < 0:
        return 0.0
    return math.fsum(math.comb(i, j) * p ** j * (1.0 - p) ** (i - j) for j in range(min(x, i) + 1))


def eq1(k, b, kb):
    """Eq. (1): expected recall under uniformly spread top values."""
    terms = [binom_cdf(kb - 1, i, 1.0 / b) for i in range(kb, k)]
    return (min(kb, k) + math.fsum(terms)) / k


def _log_comb(a, c):
    if c < 0 or c > a:
        return -math.inf
    return math.lgamma(a + 1) - math.lgamma(c + 1) - math.lgamma(a - c + 1)


def _hypergeom_cdf(x, pop, succ, draws):
    """P(X <= x), X ~ Hypergeometric(population pop, successes succ, draws)."""
    lo = max(0, draws - (pop - succ))
    total = _log_comb(pop, draws)
    terms = []
    for j in range(lo, min(x, succ, draws) + 1):
        terms.append(math.exp(_log_comb(succ, j) + _log_comb(pop - succ, draws - j) - total))
    return math.fsum(terms)


def eq1_finite(n, k, b, kb):
    """Exact expected stage-1 recall for an iid row of n distinct values in
    b interleaved buckets (finite-n reading of Eq. (1), see the module
    docstring)."""
    lo, big = n // b, n % b
    sizes = [(lo + 1, big * (lo + 1) / n), (lo, (b - big) * lo / n)]
    terms = [w * _hypergeom_cdf(kb - 1, n - 1, s - 1, i) for s, w in sizes if w > 0 for i in range(k)]
    return math.fsum(terms) / k


def eq2(n, k, b, kb):
    """Worst-case recall (reading of Eq. (2)): the top k values fill
    ceil(k / s) = ceil(b k / n) buckets, s = n / b."""
    assert n % b == 0
    s = n // b
    assert 1 <= kb <= s and 1 <= k <= n
    return (kb * (k // s) + min(kb, k % s)) / k
