"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than its own formula:
closed forms, exact rational arithmetic, a rank-count brute force that shares
nothing with sorting, the pages' invariants (blocked fold = full sort up to
tie order; sparse gathered attention = dense boolean-masked attention), and
special cases that reduce to library routines (numpy lexsort, torch's
scaled_dot_product_attention, scipy's logsumexp).
"""
import math

import numpy as np
import pytest

import dsa_inputs as di
from oracle import brute

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def bf(x):
    return di.f32_to_bf16_bits(np.asarray(x, np.float32))


# ------------------------------------------------------------------ inputs

def test_bf16_rounding_matches_torch():
    import torch

    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 37,
                        np.array([1.00390625, 1.01171875, -0.0, 0.0, 65504.0], np.float32)])
    ours = di.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------------ scores

def test_score_closed_form_two_heads(oracle_mod):
    # head 0 reads k[0], head 1 reads k[1]; w = (+1/2, -1/4): score = relu(a)/2 - relu(b)/4
    q = bf([[1, 0, 0, 0], [0, 1, 0, 0]])
    w = np.array([0.5, -0.25], np.float32)
    for a, b in [(3, 5), (-3, 5), (3, -5), (-3, -5), (0, 0), (2.5, 7)]:
        k = bf([a, b, 11, -13])
        expect = max(a, 0) * 0.5 - max(b, 0) * 0.25
        assert oracle_mod.score(q, k, w) == expect


def test_relu_is_per_head_not_on_the_sum(oracle_mod):
    q = bf([[1, 0], [0, 1]])
    k = bf([3, -5])
    w = np.array([1.0, 1.0], np.float32)
    # per-head ReLU: 3 + 0 = 3; ReLU of the weighted sum would be 0; no ReLU -2
    assert oracle_mod.score(q, k, w) == 3.0


def test_zero_query_gives_positive_zero(oracle_mod):
    q = bf(np.zeros((32, 128)))
    k = bf(np.random.default_rng(0).standard_normal(128))
    w = -np.ones(32, np.float32)
    s = oracle_mod.score(q, k, w)
    assert s == 0.0 and math.copysign(1.0, s) == 1.0


def test_head_dots_layout(oracle_mod):
    # q is [head][dim]: head h picks dimension h
    H, d = 4, 8
    q = np.zeros((H, d), np.float32)
    for h in range(H):
        q[h, h] = 1.0
    k = np.arange(1, d + 1, dtype=np.float32)
    out = oracle_mod.head_dots(bf(q), bf(k))
    assert list(out) == [1.0, 2.0, 3.0, 4.0]


def test_score_matches_exact_rationals(oracle_mod):
    """fp64 canonical score vs exact rational score on bf16 Gaussian data.

    The per-head dot products of bf16 values are exact in fp64 here (the
    exponent spread is far below 53 bits); only the 32 weighted products and
    their running sum round, so |error| <= 64 * 2^-53 * sum_h |w_h r_h|.
    """
    rng = np.random.default_rng(11)
    for _ in range(6):
        q = bf(rng.standard_normal((32, 128)))
        k = bf(rng.standard_normal(128))
        w = (rng.standard_normal(32) / math.sqrt(32)).astype(np.float32)
        got = oracle_mod.score(q, k, w)
        exact = brute.exact_score(q, k, w)
        dots = oracle_mod.head_dots(q, k)
        mag = float(np.sum(np.abs(w.astype(np.float64)) * np.maximum(dots, 0)))
        assert abs(got - float(exact)) <= 64 * 2.0 ** -53 * mag + 1e-300


def test_integer_scores_are_exact(oracle_mod):
    wl = di.CONFIGS["C0"]
    q, k, w = di.make_indexer_inputs(wl)
    for t, s in [(0, 0), (5, 17), (127, 2047), (64, 1000)]:
        assert oracle_mod.score(q[t], k[s], w[t]) == float(brute.exact_score(q[t], k[s], w[t]))


def test_row_scores_match_exact_rationals_and_stop_at_the_position(oracle_mod):
    """oracle.scores: every causal key's score equals the exact rational score; keys after
    the row's position are NaN."""
    rng = np.random.default_rng(21)
    L, N, H, d, q_pos0 = 3, 12, 4, 6, 8
    q = bf(rng.integers(-3, 4, size=(L, H, d)))
    k = bf(rng.standard_normal((N, d)))
    w = rng.choice(np.array([-0.25, 0.125, 0.5], np.float32), size=(L, H))
    got = oracle_mod.scores(q, k, w, q_pos0)
    for t in range(L):
        p = q_pos0 + t
        for s in range(N):
            if s <= p:
                assert got[t, s] == float(brute.exact_score(q[t], k[s], w[t]))
            else:
                assert np.isnan(got[t, s])
    sub = oracle_mod.scores(q, k, w, q_pos0, rows=np.array([2, 0]))
    assert np.array_equal(sub, got[[2, 0]], equal_nan=True)


# ------------------------------------------------------------------ top-k

def _tiny_case(rng, L, N, H, d, lo, hi):
    q = bf(rng.integers(lo, hi + 1, size=(L, H, d)))
    k = bf(rng.integers(lo, hi + 1, size=(N, d)))
    w = rng.choice(np.array([-0.25, -0.125, 0.125, 0.25, 0.5], np.float32), size=(L, H))
    return q, k, w


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_rank_count_bruteforce(oracle_mod, seed):
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(8, 40))
    L = int(rng.integers(1, 6))
    k = int(rng.integers(1, 9))
    lo, hi = (-1, 1) if seed % 2 == 0 else (-4, 4)  # even seeds: heavy ties
    q, kk, w = _tiny_case(rng, L, N, 4, 6, lo, hi)
    q_pos0 = int(rng.integers(0, N - L + 1))
    got = oracle_mod.topk(q, kk, w, q_pos0, k)
    want = brute.brute_topk(q, kk, w, q_pos0, k)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("block", [4096, 64, 1, 7, 2048])
def test_blocked_fold_equals_full_sort_c0(oracle_mod, block):
    wl = di.CONFIGS["C0"]
    q, k, w = di.make_indexer_inputs(wl)
    rows = np.arange(0, wl.L, 9)
    full = oracle_mod.topk(q, k, w, wl.pos0, wl.top_k, rows=rows)
    blk = oracle_mod.topk(q, k, w, wl.pos0, wl.top_k, block=block, rows=rows)
    assert np.array_equal(full, blk)


def test_blocked_fold_equals_full_sort_gaussian(oracle_mod):
    wl = di.Workload("g", 3000, 16, 300, 16, 7, "gauss")
    q, k, w = di.make_indexer_inputs(wl)
    full = oracle_mod.topk(q, k, w, wl.pos0, wl.top_k)
    for block in (4096, 512, 33):
        assert np.array_equal(full, oracle_mod.topk(q, k, w, wl.pos0, wl.top_k, block=block))


def test_single_head_is_textbook_inner_product_topk(oracle_mod):
    rng = np.random.default_rng(3)
    N, L, d, k = 300, 4, 16, 20
    q = bf(rng.standard_normal((L, 1, d)))
    kk = bf(rng.standard_normal((N, d)))
    w = np.ones((L, 1), np.float32)
    got = oracle_mod.topk(q, kk, w, N - L, k)
    qf = di.bf16_bits_to_f32(q).astype(np.float64)[:, 0]
    kf = di.bf16_bits_to_f32(kk).astype(np.float64)
    for t in range(L):
        p = N - L + t
        s = np.maximum(kf[: p + 1] @ qf[t], 0.0)
        order = np.lexsort((np.arange(p + 1), -s))  # score desc, index asc
        assert np.array_equal(got[t], np.sort(order[:k]))


def test_zero_query_selects_lowest_indices(oracle_mod):
    wl = di.Workload("z", 500, 6, 40, 16, 1, "zero")
    q, k, w = di.make_indexer_inputs(wl)
    got = oracle_mod.topk(q, k, w, wl.pos0, wl.top_k)
    assert np.array_equal(got, np.tile(np.arange(40, dtype=np.int32), (6, 1)))


def test_short_causal_rows_select_everything_then_minus_one(oracle_mod):
    wl = di.Workload("e", 64, 64, 16, 16, 2, "gauss", q_pos0=0)
    q, k, w = di.make_indexer_inputs(wl)
    got = oracle_mod.topk(q, k, w, 0, 16)
    for t in range(16):
        assert list(got[t, : t + 1]) == list(range(t + 1))
        assert (got[t, t + 1:] == -1).all()
    assert (got[16:] >= 0).all()
    for t in range(16, 64):
        assert got[t].max() <= t and len(set(got[t])) == 16


def test_top_k_larger_than_cache(oracle_mod):
    wl = di.Workload("b", 40, 4, 64, 16, 3, "gauss")
    q, k, w = di.make_indexer_inputs(wl)
    got = oracle_mod.topk(q, k, w, wl.pos0, 64)
    for t in range(4):
        p = wl.pos0 + t
        assert list(got[t, : p + 1]) == list(range(p + 1)) and (got[t, p + 1:] == -1).all()


def test_causal_mask_properties(oracle_mod):
    rng = np.random.default_rng(9)
    L, N, k, q_pos0 = 20, 100, 12, 50
    idx = rng.integers(-1, N, size=(L, k)).astype(np.int32)
    m = oracle_mod.causal_mask(idx, q_pos0)
    pos = q_pos0 + np.arange(L)[:, None]
    assert np.array_equal(m[idx <= pos], idx[idx <= pos])
    assert (m[idx > pos] == -1).all()
    assert np.array_equal(oracle_mod.causal_mask(m, q_pos0), m)


# ------------------------------------------------------------------ attention

def _attn_case(rng, L, N, H, k, q_pos0, scale_q=1.0 / 24, scale_kv=1.0 / 24):
    q = bf(rng.standard_normal((L, H, 576)) * scale_q)
    kv = bf(rng.standard_normal((N, 576)) * scale_kv)
    idx = di.random_topk_indices(rng, L, N, k, q_pos0)
    return q, kv, idx


@pytest.mark.parametrize("sharp", [False, True])
def test_sparse_equals_dense_masked(oracle_mod, sharp):
    rng = np.random.default_rng(21)
    L, N, H, k = 5, 300, 16, 40
    sq, skv = (2.0, 1.0) if sharp else (1 / 24, 1 / 24)
    q, kv, idx = _attn_case(rng, L, N, H, k, N - L, sq, skv)
    idx[1, 3] = -1
    o_s, l_s = oracle_mod.attention(q, kv, idx, N - L, di.SOFTMAX_SCALE)
    o_d, l_d = oracle_mod.attention(q, kv, idx, N - L, di.SOFTMAX_SCALE, dense=True)
    assert np.max(np.abs(o_s - o_d)) <= 1e-12
    assert np.max(np.abs(l_s - l_d)) <= 1e-12


def test_all_causal_keys_is_textbook_causal_attention(oracle_mod):
    import torch

    rng = np.random.default_rng(4)
    L, N, H = 6, 40, 16
    q_pos0 = N - L
    k = N  # every causal key selected
    q = bf(rng.standard_normal((L, H, 576)))
    kv = bf(rng.standard_normal((N, 576)) * 0.5)
    idx = np.full((L, k), -1, np.int32)
    for t in range(L):
        idx[t, : q_pos0 + t + 1] = np.arange(q_pos0 + t + 1)
    out, lse = oracle_mod.attention(q, kv, idx, q_pos0, di.SOFTMAX_SCALE)
    qt = torch.from_numpy(di.bf16_bits_to_f32(q).astype(np.float64)).permute(1, 0, 2)[None]
    kt = torch.from_numpy(di.bf16_bits_to_f32(kv).astype(np.float64))[None, None].expand(1, H, N, 576)
    vt = kt[..., :512]
    mask = torch.from_numpy(np.arange(N)[None, :] <= (q_pos0 + np.arange(L))[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                           scale=di.SOFTMAX_SCALE)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12
    from scipy.special import logsumexp

    for t in range(L):
        lg = (di.bf16_bits_to_f32(kv).astype(np.float64)[: q_pos0 + t + 1] @
              di.bf16_bits_to_f32(q).astype(np.float64)[t].T) * di.SOFTMAX_SCALE
        assert np.max(np.abs(lse[t] - logsumexp(lg, axis=0))) < 1e-12


def test_single_key_returns_that_latent_row(oracle_mod):
    rng = np.random.default_rng(8)
    L, N, H = 4, 50, 16
    q, kv, _ = _attn_case(rng, L, N, H, 1, N - L)
    idx = rng.integers(0, N - L, size=(L, 1)).astype(np.int32)
    out, lse = oracle_mod.attention(q, kv, idx, N - L, di.SOFTMAX_SCALE)
    lat = di.bf16_bits_to_f32(kv).astype(np.float64)
    for t in range(L):
        assert np.array_equal(out[t], np.broadcast_to(lat[idx[t, 0], :512], (H, 512)))
        lg = di.bf16_bits_to_f32(q).astype(np.float64)[t] @ lat[idx[t, 0]] * di.SOFTMAX_SCALE
        assert np.max(np.abs(lse[t] - lg)) < 1e-14


def test_zero_query_gives_mean_and_log_count(oracle_mod):
    rng = np.random.default_rng(12)
    L, N, H, k = 3, 80, 16, 10
    _, kv, idx = _attn_case(rng, L, N, H, k, N - L)
    idx[2, :4] = -1
    q = np.zeros((L, H, 576), np.uint16)
    out, lse = oracle_mod.attention(q, kv, idx, N - L, di.SOFTMAX_SCALE)
    lat = di.bf16_bits_to_f32(kv).astype(np.float64)[:, :512]
    for t in range(L):
        v = idx[t][idx[t] >= 0]
        assert np.max(np.abs(out[t] - lat[v].mean(0))) < 1e-15
        assert np.allclose(lse[t], math.log(len(v)), rtol=0, atol=1e-15)


def test_identical_rows_return_that_row(oracle_mod):
    rng = np.random.default_rng(13)
    L, N, H, k = 2, 30, 16, 8
    q = bf(rng.standard_normal((L, H, 576)))
    row = bf(rng.standard_normal(576))
    kv = np.tile(row, (N, 1))
    idx = di.random_topk_indices(rng, L, N, k, N - L)
    out, _ = oracle_mod.attention(q, kv, idx, N - L, di.SOFTMAX_SCALE)
    assert np.max(np.abs(out - di.bf16_bits_to_f32(row)[:512].astype(np.float64))) < 1e-15


def test_empty_row_gives_zero_and_minus_inf(oracle_mod):
    rng = np.random.default_rng(14)
    L, N, H, k = 2, 30, 16, 8
    q, kv, idx = _attn_case(rng, L, N, H, k, N - L)
    idx[0, :] = -1
    out, lse = oracle_mod.attention(q, kv, idx, N - L, di.SOFTMAX_SCALE)
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all()
    assert np.isfinite(lse[1]).all()


def test_minus_one_and_future_indices_are_skipped(oracle_mod):
    rng = np.random.default_rng(15)
    L, N, H, k = 4, 200, 16, 30
    q_pos0 = 100
    q, kv, idx = _attn_case(rng, L, N, H, k, q_pos0)
    noisy = idx.copy()
    noisy[:, ::5] = -1
    noisy[:, 1::7] = N - 1  # future for every row
    clean = oracle_mod.causal_mask(noisy, q_pos0)
    a = oracle_mod.attention(q, kv, noisy, q_pos0, di.SOFTMAX_SCALE)
    b = oracle_mod.attention(q, kv, clean, q_pos0, di.SOFTMAX_SCALE)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------------ vector retrieval (inner-product top-k)

def test_retrieval_integer_scores_match_integer_matmul(oracle_mod):
    """Small integers: every fp64 partial sum is exact, so the scores are numpy's int64
    matmul and the selection is a lexsort on (score desc, index asc)."""
    rng = np.random.default_rng(21)
    M, N, d, k = 5, 700, 128, 37
    qi = rng.integers(-6, 7, size=(M, d))
    xi = rng.integers(-6, 7, size=(N, d))
    got, kth = oracle_mod.retrieval_topk(bf(qi), bf(xi), k, return_kth=True)
    s = qi.astype(np.int64) @ xi.astype(np.int64).T
    for t in range(M):
        order = np.lexsort((np.arange(N), -s[t]))
        assert np.array_equal(got[t], np.sort(order[:k]))
        assert kth[t] == s[t, order[k - 1]]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_retrieval_matches_rank_count_with_exact_rationals(oracle_mod, seed):
    """Gaussian bf16 rows of 16 dims: the fp64 sums are exact, so exact rational scores
    plus the rank-count rule (no sorting) must give the same selection."""
    from fractions import Fraction

    rng = np.random.default_rng(100 + seed)
    M, N, d, k = 3, 40, 16, 9
    q = bf(rng.standard_normal((M, d)))
    x = bf(rng.standard_normal((N, d)))
    qf, xf = di.bf16_bits_to_f32(q), di.bf16_bits_to_f32(x)
    got = oracle_mod.retrieval_topk(q, x, k)
    for t in range(M):
        scores = [sum((Fraction(float(qf[t, i])) * Fraction(float(xf[j, i])) for i in range(d)), Fraction(0))
                  for j in range(N)]
        assert got[t].tolist() == brute.rank_count_topk(scores, N - 1, k)


def test_retrieval_equals_two_head_indexer_form(oracle_mod):
    """ReLU(s) - ReLU(-s) = s: the indexer score with heads (q, -q), weights (1, -1) and
    zero heads elsewhere is the inner product, in the canonical fp64 order too."""
    rng = np.random.default_rng(22)
    M, N, d, k = 4, 3000, 128, 256
    q = bf(rng.standard_normal((M, d)))
    x = bf(rng.standard_normal((N, d)))
    got = oracle_mod.retrieval_topk(q, x, k)
    for t in range(M):
        qe = np.zeros((1, 32, d), np.uint16)
        qe[0, 0] = q[t]
        qe[0, 1] = q[t] ^ np.uint16(0x8000)  # bf16 negation
        w = np.zeros((1, 32), np.float32)
        w[0, 0], w[0, 1] = 1.0, -1.0
        assert np.array_equal(got[t], oracle_mod.topk(qe, x, w, N - 1, k)[0])


def test_retrieval_negative_scores_are_ranked_not_clipped(oracle_mod):
    """q = -x_0 makes every score of a unit-norm-ish corpus negative for most rows: the
    top-k must follow the signed score (no ReLU), which the indexer's form would clip."""
    rng = np.random.default_rng(23)
    N, d, k = 200, 32, 10
    x = bf(np.abs(rng.standard_normal((N, d))))
    q = bf(-np.ones((1, d)))
    got = oracle_mod.retrieval_topk(q, x, k)[0]
    s = -di.bf16_bits_to_f32(x).astype(np.float64).sum(axis=1)
    order = np.lexsort((np.arange(N), -s))
    assert np.array_equal(got, np.sort(order[:k]))
    assert not np.array_equal(got, np.arange(k))  # what clipping every score to 0 would give


def test_retrieval_ties_and_small_corpus(oracle_mod):
    x = np.tile(bf(np.ones((1, 8))), (50, 1))
    q = bf(np.ones((2, 8)))
    assert np.array_equal(oracle_mod.retrieval_topk(q, x, 7), np.tile(np.arange(7), (2, 1)))
    got = oracle_mod.retrieval_topk(q, x[:5], 8)
    assert np.array_equal(got, np.tile([0, 1, 2, 3, 4, -1, -1, -1], (2, 1)))


def test_dot_is_left_to_right_and_positive_zero(oracle_mod):
    """2^60 + 1 - 2^60 is 0 left to right (the 1 is absorbed), 1 exactly: the canonical
    order is the sequential one.  A negative-zero sum becomes +0."""
    a = bf([2.0 ** 60, 1.0, -(2.0 ** 60)])
    one = bf([1.0, 1.0, 1.0])
    assert oracle_mod.dot(a, one) == 0.0
    assert oracle_mod.dot(bf([2.0 ** 60, -(2.0 ** 60), 1.0]), one) == 1.0
    z = oracle_mod.dot(bf([-1.0]), bf([0.0]))
    assert z == 0.0 and math.copysign(1.0, z) == 1.0
