"""Top-K sparse-attention decode, dense-then-masked, in float64 (CPU).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* "Recall Before You Rank ..." (fugumt page), Abstract: the query is scored
  against the full KV cache, a global Top-K is selected, and softmax and value
  aggregation run over only that subset.
* STARC (Pith review page), Figure 3 caption: per head q in R^{1 x d_h} and
  K, V in R^{L x d_h}.
* "Approximate Top-k for Increased Parallelism" (Pith review page), "What
  carries the argument": the bucketed selection that may replace the exact
  Top-K.

Readings (the pages leave these open):
* score s_j = scale * <q, K_j> with scale = 1/sqrt(d_h); no causal mask at
  decode, every one of the L cached keys is a candidate.
* Softmax is normalised over the selected set only, with the maximum
  subtracted; masking the rest to -inf and running a dense softmax over all L
  is the same thing, and is what is written here.
* Grouped-query heads: query head h reads KV head h // (H_q / H_kv), and
  every query head selects its own Top-K.
* Selected indices are reported by score descending, then index ascending.
* Candidate rerank ("Recall Before You Rank ...", Abstract: the supports of
  the most similar cached queries are united with a recent window, and only
  that compact candidate set is reranked with exact current-query scores):
  the candidate set is the union, as a set, of the given indices that lie in
  [0, L) and the last `window` positions; the Top-K is exact within it, and a
  set smaller than K is attended whole.
"""

import numpy as np

from .topk import bucketed_topk, exact_topk


def bf16_bits_to_f64(bits):
    bits = np.asarray(bits)
    assert bits.dtype == np.uint16
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_scores(q_bits, k_bits, scale, hkv=None):
    """s[b, h, j] = scale * sum_d q[b, h, d] * K[b, h // g, j, d] in float64.

    q_bits: [B, Hq, D] bf16 bit patterns; k_bits: [B, Hkv, L, D].
    """
    q = bf16_bits_to_f64(q_bits)
    kk = bf16_bits_to_f64(k_bits)
    bsz, hq, d = q.shape
    hkv = kk.shape[1]
    g = hq // hkv
    assert g * hkv == hq
    s = np.empty((bsz, hq, kk.shape[2]), dtype=np.float64)
    for bi in range(bsz):
        for h in range(hq):
            s[bi, h] = kk[bi, h // g] @ q[bi, h]
    return s * float(scale)


def select(scores_row_block, k_sel, b, kb):
    """Top-K selection over score rows [R, L]: exact when (b, kb) = (1, K),
    else bucketed with a final exact Top-K (which only sorts when
    b * kb == K).  Returns indices [R, K]."""
    if b == 1 and kb == k_sel:
        idx, _ = exact_topk(scores_row_block, k_sel, dtype="f64")
    else:
        idx, _ = bucketed_topk(scores_row_block, k_sel, b, kb, True, dtype="f64")
    return idx


def softmax_v_subset(s_row, idx, v_rows):
    """Dense-then-masked softmax(s) @ V over the index set idx, float64.

    s_row: [L] scores; idx: selected positions; v_rows: [L, D] float64."""
    masked = np.full(s_row.shape, -np.inf)
    masked[idx] = s_row[idx]
    mx = masked.max()
    w = np.exp(masked - mx)  # exp(-inf) = 0 outside the subset
    p = w / w.sum()
    return p @ v_rows


def attn_decode(q_bits, k_bits, v_bits, scale, k_sel, b, kb, scores=None):
    """Reference decode step.  Returns (out [B, Hq, D] float64,
    sel_idx [B, Hq, K] int64, scores [B, Hq, L] float64).

    `scores` may be passed in (for example fp32 scores to check a selection
    made on them); otherwise they are computed in float64."""
    if scores is None:
        scores = decode_scores(q_bits, k_bits, scale)
    vv = bf16_bits_to_f64(v_bits)
    bsz, hq, length = scores.shape
    hkv = vv.shape[1]
    g = hq // hkv
    out = np.empty((bsz, hq, vv.shape[3]), dtype=np.float64)
    sel = np.empty((bsz, hq, k_sel), dtype=np.int64)
    for bi in range(bsz):
        sel[bi] = select(np.asarray(scores[bi], dtype=np.float64), k_sel, b, kb)
        for h in range(hq):
            out[bi, h] = softmax_v_subset(np.asarray(scores[bi, h], dtype=np.float64), sel[bi, h], vv[bi, h // g])
    return out, sel, scores


def rerank_candidates(cand_row, window, length):
    """The candidate set of one head: the given indices inside [0, L) united
    with the last `window` positions, as a sorted array without repeats."""
    c = set(int(j) for j in np.asarray(cand_row).ravel() if 0 <= int(j) < length)
    c.update(range(length - window, length))
    return np.array(sorted(c), dtype=np.int64)


def rerank_decode(q_bits, k_bits, v_bits, scale, cand, window, k_sel, scores=None):
    """Reference candidate-rerank decode step.  cand: [B, Hq, C] indices per
    query head (entries outside [0, L) are ignored).  Returns (out [B, Hq, D]
    float64, sel [B, Hq, K] int64 padded with -1 when a candidate set holds
    fewer than K keys, scores [B, Hq, L] float64)."""
    if scores is None:
        scores = decode_scores(q_bits, k_bits, scale)
    vv = bf16_bits_to_f64(v_bits)
    bsz, hq, length = scores.shape
    g = hq // vv.shape[1]
    out = np.empty((bsz, hq, vv.shape[3]), dtype=np.float64)
    sel = np.full((bsz, hq, k_sel), -1, dtype=np.int64)
    for bi in range(bsz):
        for h in range(hq):
            c = rerank_candidates(cand[bi, h], window, length)
            s_row = np.asarray(scores[bi, h], dtype=np.float64)
            kk = min(k_sel, len(c))
            top, _ = exact_topk(s_row[c][None, :], kk, dtype="f64")
            chosen = c[top[0]]
            sel[bi, h, :kk] = chosen
            out[bi, h] = softmax_v_subset(s_row, chosen, vv[bi, h // g])
    return out, sel, scores
