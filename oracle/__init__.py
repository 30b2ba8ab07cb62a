"""CPU oracle for top-k selection and top-K sparse-attention decode.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, deliberately
obvious reference written from the method's definition on the pages:

* "Approximate Top-k for Increased Parallelism" (Pith review page):
  "What carries the argument" (the two-stage bucketed top-k, Eq. (1) and the
  description of Eq. (2)), "What would settle it" (one residue class modulo b),
  Figures 6 and 8 captions (contiguous against interleaved assignment),
  Figure 2 caption (n = 11, k = 4, b = 3, k_b = 2 toy) and Figure 12 caption
  (ties at the k-th value need a "collect" step).
* "Recall Before You Rank: Similarity-Guided Top-K Reuse ..." (fugumt page),
  Abstract: Top-K sparse attention scores the current query against the full
  KV cache, takes a global Top-K, and does softmax and value aggregation over
  that subset only; ReTopK reranks a compact candidate set (retrieved
  supports united with a recent window) with exact current-query scores.
* STARC (Pith review page), Figure 3 caption: q in R^{1 x d_h}, K, V in
  R^{L x d_h} per head.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library and the
library never imports it.  Floating point work is done in float64.
"""

from .topk import (  # noqa: F401
    to_f64,
    exact_topk,
    bucketed_topk,
    bucket_members,
    contiguous_members,
)
from .recall import (  # noqa: F401
    recall,
    recall_by_bucket_counts,
    value_recall,
    binom_cdf,
    eq1,
    eq1_finite,
    eq2,
)
from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    decode_scores,
    attn_decode,
    softmax_v_subset,
    rerank_candidates,
    rerank_decode,
)
