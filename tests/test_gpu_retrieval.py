"""GPU parity of dsa_retrieval_topk (inner-product top-k over a corpus) against the
oracle: selected corpus rows must be bit-exact (score desc, lower row first, ascending
output, -1 padding).

Inputs: Gaussian queries and corpus rows, a concentrated corpus (rows close to one common
direction: scores crowd into a narrow range, the LiteTopK page's score concentration), small
integers (many exactly equal scores: the tie rule decides), and elements scaled by 2^±24
(dot products that need more than 53 bits: the sequential fp64 re-score).
"""
import numpy as np
import pytest

import dsa_inputs as di
from tests.gpu_util import report, to_dev_bf16

pytestmark = pytest.mark.gpu


def make(M, N, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "int":
        q = rng.integers(-3, 4, size=(M, 128)).astype(np.float32)
        x = rng.integers(-3, 4, size=(N, 128)).astype(np.float32)
    elif kind == "concentrated":
        q = rng.standard_normal((M, 128), dtype=np.float32)
        c = rng.standard_normal(128, dtype=np.float32)
        x = 0.9 * c[None, :] + 0.1 * rng.standard_normal((N, 128), dtype=np.float32)
    elif kind == "wide":
        q = rng.standard_normal((M, 128), dtype=np.float32) * np.exp2(rng.integers(-24, 25, size=(M, 128)))
        x = rng.standard_normal((N, 128), dtype=np.float32) * np.exp2(rng.integers(-24, 25, size=(N, 128)))
    else:
        q = rng.standard_normal((M, 128), dtype=np.float32)
        x = rng.standard_normal((N, 128), dtype=np.float32)
    return di.f32_to_bf16_bits(q.astype(np.float32)), di.f32_to_bf16_bits(x.astype(np.float32))


def run_gpu(dsa, q, x, k, q_block=1024):
    import torch

    out = dsa.retrieval_topk(to_dev_bf16(q), to_dev_bf16(x), k, q_block=q_block)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(oracle_mod, got, q, x, k, rows=None, what=""):
    want = oracle_mod.retrieval_topk(q, x, k, rows=rows)
    sub = got if rows is None else got[rows]
    bad = np.nonzero((sub != want).any(axis=1))[0]
    assert bad.size == 0, f"{what}: {bad.size} rows differ, first {bad[0] if rows is None else rows[bad[0]]}"
    report(f"{what}: {sub.shape[0]} rows bit-exact")


@pytest.mark.parametrize("kind", ["gauss", "concentrated", "int"])
def test_ragged_sizes_match_oracle(dsa_gpu, oracle_mod, kind):
    """M = 300 (two query groups and a ragged one), N = 50,001 (a ragged last tile)."""
    q, x = make(300, 50001, kind, 1)
    got = run_gpu(dsa_gpu, q, x, 256)
    check(oracle_mod, got, q, x, 256, what=f"retrieval {kind}")
    assert (np.diff(got, axis=1) > 0).all()


@pytest.mark.parametrize("k", [1, 100, 2048, 4096])
def test_top_k_values(dsa_gpu, oracle_mod, k):
    q, x = make(40, 20000, "gauss", 2)
    check(oracle_mod, run_gpu(dsa_gpu, q, x, k), q, x, k, what=f"k={k}")


@pytest.mark.parametrize("N", [1, 31, 33, 700, 2048])
def test_small_corpus(dsa_gpu, oracle_mod, N):
    """N <= top_k returns every row then -1; just above it the whole corpus is scored."""
    q, x = make(9, N, "gauss", 3)
    check(oracle_mod, run_gpu(dsa_gpu, q, x, 700), q, x, 700, what=f"N={N}")


def test_wide_dynamic_range(dsa_gpu, oracle_mod):
    q, x = make(16, 6000, "wide", 4)
    check(oracle_mod, run_gpu(dsa_gpu, q, x, 64), q, x, 64, what="wide")


def test_query_block_invariance(dsa_gpu):
    q, x = make(260, 30000, "concentrated", 5)
    ref = run_gpu(dsa_gpu, q, x, 512)
    for qb in (64, 100, 7):
        assert np.array_equal(ref, run_gpu(dsa_gpu, q, x, 512, q_block=qb)), qb


def test_forced_fallback_fold(dsa_gpu, oracle_mod, monkeypatch):
    q, x = make(20, 15000, "gauss", 6)
    normal = run_gpu(dsa_gpu, q, x, 300)
    monkeypatch.setenv("DSA_DEBUG_FORCE_FALLBACK", "1")
    forced = run_gpu(dsa_gpu, q, x, 300)
    monkeypatch.delenv("DSA_DEBUG_FORCE_FALLBACK")
    assert np.array_equal(normal, forced)
    check(oracle_mod, forced, q, x, 300, what="fold")


def test_bench_size_sampled_rows(dsa_gpu, oracle_mod):
    """1,024 queries over a 1,048,576-row corpus, top_k 1,024 (the bench workload), on
    sampled rows the oracle computes one by one."""
    q, x = make(1024, 1 << 20, "gauss", 7)
    got = run_gpu(dsa_gpu, q, x, 1024)
    rows = np.array([0, 1, 127, 128, 511, 640, 1000, 1023], dtype=np.int64)
    check(oracle_mod, got, q, x, 1024, rows=rows, what="1M corpus")
    assert (np.diff(got, axis=1) > 0).all() and (got >= 0).all()
