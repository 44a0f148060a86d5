"""GPU tests of the selection's less common paths, against the oracle.

- top_k between 2,048 and 4,096: the select kernel then runs a block size that does not
  divide its 2,048 histogram bins (576 .. 960 threads); every bin must still be counted,
  so rows finish on the candidate path instead of falling back.
- Scores spread over many scales (zeros, 2^-100, 2^-66, 2^-33, values near 1): value
  binning cannot isolate the k-th score in three levels.  Select still bounds it by the
  narrowest bin's range and ranks that band exactly when it fits its buffer; otherwise the
  row goes to the blocked fold, whose k-th search finishes with the exact radix select.

- Scores that favour recent keys (key norms growing with position): most candidates come
  from the newest keys, and a row's list must hold them wherever they fall; no row may fall
  back to the fold for it.

The selection counters (dsa_indexer_topk_stats) show which path each row took.
"""
import numpy as np
import pytest

import dsa_inputs as di
from tests.gpu_util import report, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def run_with_stats(dsa, q, k, w, q_pos0, top_k, q_block=1024):
    import torch

    L, N = q.shape[0], k.shape[0]
    ws = torch.empty(dsa.workspace_bytes(L, N, top_k, q_block), dtype=torch.uint8, device="cuda:0")
    out = dsa.indexer_topk(to_dev_bf16(q), to_dev_bf16(k), to_dev(w), q_pos0, top_k, q_block=q_block,
                           workspace=ws)
    stats = dsa.indexer_stats(ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), stats


def multiscale_case(N, L, seed):
    """One live head reading key dimension 0: score(s) = ReLU(k[s, 0]).  200 keys score
    between 1 and 3 (distinct), three score 2^-33, 2^-66 and 2^-100, every other key 0."""
    rng = np.random.default_rng(seed)
    q = np.zeros((L, 32, 128), np.float32)
    q[:, 0, 0] = 1.0
    w = np.zeros((L, 32), np.float32)
    w[:, 0] = 1.0
    k = np.zeros((N, 128), np.float32)
    vals = np.concatenate([1.0 + np.arange(128) / 128.0, 2.0 + np.arange(72) / 32.0]).astype(np.float32)
    big = rng.choice(N - L - 16, size=vals.size, replace=False)
    k[big, 0] = vals
    tiny = rng.choice(np.setdiff1d(np.arange(N - L), big), size=3, replace=False)
    k[tiny, 0] = np.array([2.0 ** -33, 2.0 ** -66, 2.0 ** -100], np.float32)
    # other dimensions of the keys carry values the live head does not read
    k[:, 1:] = rng.integers(-2, 3, size=(N, 127))
    return di.f32_to_bf16_bits(q), di.f32_to_bf16_bits(k), w


def test_multiscale_scores_in_select(dsa_gpu, oracle_mod):
    """Every causal key is a candidate (N below the candidate capacity).  Three levels of
    bins leave the k-th score (0) in a bin that still holds the zeros and 2^-100; widened by
    2 delta, the band is the zeros and the three tiny scores (about 800 entries), which
    select re-scores in fp64 (2^-100 takes the sequential evaluation) and ranks."""
    N, L, top_k = 1000, 8, 256
    q, k, w = multiscale_case(N, L, 1)
    got, st = run_with_stats(dsa_gpu, q, k, w, N - L, top_k)
    report(f"multiscale select: {st}")
    want = oracle_mod.topk(q, k, w, N - L, top_k)
    assert np.array_equal(got, want)
    assert st["rows"] == L and st["rows_fallback"] == 0 and st["rows_failed"] == 0
    assert st["band_max"] >= 790


def test_multiscale_scores_radix_in_fold(dsa_gpu, oracle_mod):
    """The same scores over 7,000 keys: about 6,800 keys lie within the error bound of the k-th
    score, far more than select's band buffer, so the rows go to the blocked fold, whose k-th
    searches need the radix pass."""
    N, L, top_k = 7000, 8, 2048
    q, k, w = multiscale_case(N, L, 2)
    got, st = run_with_stats(dsa_gpu, q, k, w, N - L, top_k)
    report(f"multiscale fold: {st}")
    want = oracle_mod.topk(q, k, w, N - L, top_k)
    assert np.array_equal(got, want)
    assert st["rows_fallback"] == L and st["fallback_band"] == L and st["kth_radix"] == L
    assert st["rows_failed"] == 0


@pytest.mark.parametrize("top_k", [2049, 3000, 3840])
def test_topk_between_2048_and_4096(dsa_gpu, oracle_mod, top_k):
    """1,024 rows (128 row groups, two key halves sharing each row's list); select runs
    cap / 32 threads = 320 .. 512 (5 to 8 waves)."""
    wl = di.Workload("k3000", 60000, 1024, top_k, 16, 23, "gauss")
    q, k, w = di.make_indexer_inputs(wl)
    got, st = run_with_stats(dsa_gpu, q, k, w, wl.pos0, top_k)
    report(f"top_k {top_k}: {st}")
    rows = np.array([0, 1, 7, 8, 100, 511, 512, 700, 1015, 1023], dtype=np.int64)
    want = oracle_mod.topk(q, k, w, wl.pos0, top_k, rows=rows)
    assert np.array_equal(got[rows], want)
    assert (np.diff(got, axis=1) > 0).all()
    assert st["rows_failed"] == 0
    assert st["rows_fallback"] <= wl.L // 100, "rows should finish on the candidate path"


@pytest.mark.parametrize("N,L", [(65536, 1024), (131072, 1024)])
def test_recency_biased_scores(dsa_gpu, oracle_mod, N, L):
    """Keys scaled by 1 + s/N (the newest eighth of a row's keys holds about a quarter of its
    candidates, the newest half about three quarters): indices bit-exact on sampled rows and
    every row finished in select, none in the fold."""
    wl = di.Workload("recency", N, L, 2048, 16, 31, "recency")
    q, k, w = di.make_indexer_inputs(wl)
    got, st = run_with_stats(dsa_gpu, q, k, w, wl.pos0, wl.top_k)
    report(f"recency N={N} L={L}: {st}")
    rows = np.array([0, 1, 7, 8, 255, 511, 512, 777, 1016, 1023], dtype=np.int64)
    want = oracle_mod.topk(q, k, w, wl.pos0, wl.top_k, rows=rows)
    assert np.array_equal(got[rows], want)
    assert (np.diff(got, axis=1) > 0).all()
    assert st["rows_failed"] == 0 and st["rows_fallback"] == 0


def test_recency_biased_scores_c4_shape(dsa_gpu, oracle_mod):
    """C4's shape (786,432 keys, 8,192 queries in 8 blocks) with recency-biased keys: indices
    bit-exact on sampled rows at every block boundary and no row falls back."""
    wl = di.Workload("recency-c4", 786432, 8192, 2048, 16, 32, "recency")
    q, k, w = di.make_indexer_inputs(wl)
    got, st = run_with_stats(dsa_gpu, q, k, w, wl.pos0, wl.top_k)
    report(f"recency C4 shape: {st}")
    rows = np.array([0, 1023, 1024, 4095, 4096, 7167, 8191], dtype=np.int64)
    want = oracle_mod.topk(q, k, w, wl.pos0, wl.top_k, rows=rows)
    assert np.array_equal(got[rows], want)
    assert (np.diff(got, axis=1) > 0).all()
    assert st["rows_failed"] == 0 and st["rows_fallback"] == 0


def test_zero_rows_fold_beside_select(dsa_gpu, oracle_mod):
    """Three all-zero query rows in a block of 64 at 131,072 keys: every score of those rows is
    0, so all their keys are candidates and they fall back to the fold, whose split form (key
    ranges merged) must give keys 0 .. k-1 (the lower index wins every tie); the other rows
    finish in select in the same launches."""
    wl = di.Workload("zero-mix", 131072, 64, 2048, 16, 33, "gauss")
    q, k, w = di.make_indexer_inputs(wl)
    zero_rows = np.array([3, 17, 40])
    qf = di.bf16_bits_to_f32(q)
    qf[zero_rows] = 0.0
    q = di.f32_to_bf16_bits(qf)
    got, st = run_with_stats(dsa_gpu, q, k, w, wl.pos0, wl.top_k)
    report(f"zero rows beside select: {st}")
    assert st["rows_fallback"] == zero_rows.size and st["rows_failed"] == 0
    for r in zero_rows:
        assert np.array_equal(got[r], np.arange(wl.top_k, dtype=np.int32))
    rows = np.array([0, 2, 4, 18, 39, 41, 63], dtype=np.int64)
    want = oracle_mod.topk(q, k, w, wl.pos0, wl.top_k, rows=rows)
    assert np.array_equal(got[rows], want)
