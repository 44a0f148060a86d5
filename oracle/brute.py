"""Tiny-input brute-force definitions -- TEST INFRASTRUCTURE ONLY.

These restate the selection rule in a form that shares nothing with sorting,
to pin the C oracle:

  A causal key s of query t is selected iff fewer than k causal keys beat it,
  where x beats y when score(x) > score(y), or the scores are equal and x has
  the lower index (the tie rule; the GLM page, How it works, says the blocked
  fold picks the same keys as the full argpartition up to the order of equal
  scores, and the lower index winning makes the selected set unique).

Scores are computed with exact rationals (fractions.Fraction), valid whenever
the inputs are dyadic (bf16 and fp32 values always are), so a rounding slip in
the fp64 oracle would not hide here on exactly representable data.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def _bf16_to_fraction(b: int) -> Fraction:
    v = np.array([int(b) << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(v))


def exact_score(q_row_bits, k_row_bits, w_row) -> Fraction:
    """sum_h w_h * max(0, q_h . k) in exact rational arithmetic."""
    H, d = q_row_bits.shape
    kf = [_bf16_to_fraction(x) for x in k_row_bits]
    total = Fraction(0)
    for h in range(H):
        dot = Fraction(0)
        for i in range(d):
            dot += _bf16_to_fraction(q_row_bits[h, i]) * kf[i]
        if dot > 0:
            total += Fraction(float(w_row[h])) * dot
    return total


def rank_count_topk(scores, p: int, k: int) -> list[int]:
    """Selected keys (ascending) among 0..p by the rank-count definition."""
    sel = []
    for s in range(p + 1):
        beaten_by = 0
        for x in range(p + 1):
            if x == s:
                continue
            if scores[x] > scores[s] or (scores[x] == scores[s] and x < s):
                beaten_by += 1
        if beaten_by < k:
            sel.append(s)
    return sel


def brute_topk(q_idx, k_idx, w, q_pos0: int, top_k: int) -> np.ndarray:
    """Exact-rational scores + rank-count selection, padded with -1."""
    L = q_idx.shape[0]
    N = k_idx.shape[0]
    out = np.full((L, top_k), -1, np.int32)
    for t in range(L):
        p = min(q_pos0 + t, N - 1)
        sc = [exact_score(q_idx[t], k_idx[s], w[t]) for s in range(p + 1)]
        sel = rank_count_topk(sc, p, top_k)
        out[t, :len(sel)] = sel
    return out
