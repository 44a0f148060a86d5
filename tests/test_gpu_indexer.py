"""GPU parity of dsa_indexer_topk and dsa_causal_mask_topk against the CPU oracle.

Indices must be bit-exact.  C0 and the integer twins make fp32 scores exact; on
the Gaussian configurations exactness comes from the fp64 re-score of the
near-threshold band.  C2-C4 and their integer twins are checked end to end in
test_gpu_configs.py.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import dsa_inputs as di
from tests.gpu_util import report, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def run_gpu(dsa, q, k, w, q_pos0, top_k, q_block=1024):
    import torch

    out = dsa.indexer_topk(to_dev_bf16(q), to_dev_bf16(k), to_dev(w), q_pos0, top_k, q_block=q_block)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def sample_rows(L, n, seed=0):
    rng = np.random.default_rng(seed)
    rows = set([0, L - 1, min(L - 1, 1023), min(L - 1, 1024)])
    rows.update(rng.choice(L, size=min(L, n), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def check_rows(oracle_mod, got, q, k, w, q_pos0, top_k, rows=None, what=""):
    want = oracle_mod.topk(q, k, w, q_pos0, top_k, rows=rows)
    sub = got if rows is None else got[rows]
    bad = np.nonzero((sub != want).any(axis=1))[0]
    assert bad.size == 0, f"{what}: {bad.size} rows differ, first row {bad[0] if rows is None else rows[bad[0]]}"
    report(f"{what}: {sub.shape[0]} rows bit-exact")


def test_c0_full_bit_exact(dsa_gpu, oracle_mod):
    wl = di.CONFIGS["C0"]
    q, k, w = di.make_indexer_inputs(wl)
    got = run_gpu(dsa_gpu, q, k, w, wl.pos0, wl.top_k)
    check_rows(oracle_mod, got, q, k, w, wl.pos0, wl.top_k, what="C0")


@pytest.mark.parametrize("q_block", [128, 32, 7, 1])
def test_query_block_invariance_c0(dsa_gpu, q_block):
    wl = di.CONFIGS["C0"]
    q, k, w = di.make_indexer_inputs(wl)
    ref = run_gpu(dsa_gpu, q, k, w, wl.pos0, wl.top_k, 1024)
    got = run_gpu(dsa_gpu, q, k, w, wl.pos0, wl.top_k, q_block)
    assert np.array_equal(ref, got)


def test_integer_twin_c1_full(dsa_gpu, oracle_mod):
    wl = di.int_twin("C1")
    q, k, w = di.make_indexer_inputs(wl)
    got = run_gpu(dsa_gpu, q, k, w, wl.pos0, wl.top_k)
    check_rows(oracle_mod, got, q, k, w, wl.pos0, wl.top_k, what="C1i")


def test_c1_gaussian_full_bit_exact(dsa_gpu, oracle_mod):
    wl = di.CONFIGS["C1"]
    q, k, w = di.make_indexer_inputs(wl)
    got = run_gpu(dsa_gpu, q, k, w, wl.pos0, wl.top_k)
    check_rows(oracle_mod, got, q, k, w, wl.pos0, wl.top_k, what="C1")


# ------------------------------------------------------------------ edge cases

def test_max_topk_key_ordered(dsa_gpu, oracle_mod):
    """top_k = 4,096 over 1,024 rows (128 groups, two key halves sharing each row's list):
    the candidate capacity is 16,384, so select runs 512 threads (8 waves) through its
    bitmap output."""
    wl = di.Workload("maxk", 20000, 1024, 4096, 16, 19, "gauss")
    q, k, w = di.make_indexer_inputs(wl)
    got = run_gpu(dsa_gpu, q, k, w, wl.pos0, wl.top_k)
    rows = np.array([0, 5, 8, 300, 512, 777, 1023], dtype=np.int64)
    check_rows(oracle_mod, got, q, k, w, wl.pos0, wl.top_k, rows=rows, what="top_k 4096, 1024 rows")
    assert (np.diff(got, axis=1) > 0).all()


def test_full_candidate_lists(dsa_gpu, oracle_mod):
    """1,024 rows in 128 groups (two key halves sharing each row's list).  With N = 8,184 =
    capacity - 8 no group samples a threshold: every row keeps all of its 7,161 to 8,184
    causal keys, so the halves' runs (one from each end) fill the list almost to its 8,192
    slots."""
    wl = di.Workload("full", 8184, 1024, 2048, 16, 17, "gauss", q_pos0=8184 - 1024)
    q, k, w = di.make_indexer_inputs(wl)
    got = run_gpu(dsa_gpu, q, k, w, wl.pos0, wl.top_k)
    rows = np.array([0, 1, 7, 8, 511, 512, 1016, 1022, 1023], dtype=np.int64)
    check_rows(oracle_mod, got, q, k, w, wl.pos0, wl.top_k, rows=rows, what="full candidate lists")
    assert (np.diff(got, axis=1) > 0).all()


@pytest.mark.parametrize("case", [
    dict(N=300, L=300, top_k=64, q_pos0=0, kind="gauss"),      # early rows have < k keys (-1 tail)
    dict(N=9000, L=37, top_k=2048, q_pos0=8963, kind="gauss"),  # ragged group, just above capacity
    dict(N=5000, L=5, top_k=4096, kind="gauss"),               # maximum top_k
    dict(N=3000, L=6, top_k=3000, kind="gauss"),               # k >= every row's key count
    dict(N=20000, L=9, top_k=1, kind="sink"),                  # k = 1
    dict(N=20000, L=13, top_k=100, kind="int"),                # integer ties, small k
    dict(N=1, L=1, top_k=5, kind="gauss"),                     # single key
    dict(N=40000, L=6, top_k=2048, kind="concentrated"),
    # elements scaled by 2^-24..2^24: the dot products need more than 53 bits, so the band
    # re-score takes the sequential fp64 evaluation (in select, and in the fold when the
    # band outgrows select's buffer)
    dict(N=1000, L=8, top_k=64, kind="wide"),
    dict(N=3000, L=8, top_k=64, kind="wide"),
    # few row groups: more key parts per group, candidates appended to one list per row,
    # the selection put back in key order through a bitmap of the causal keys ...
    dict(N=131072, L=1, top_k=2048, kind="concentrated"),        # decode: 256 key parts
    dict(N=50000, L=3, top_k=512, kind="sink"),
    dict(N=20000, L=200, top_k=700, kind="gauss"),               # 25 groups: 16 key parts
    # ... or, past 262,144 causal keys, by sorting the selection
    dict(N=300000, L=2, top_k=2048, kind="gauss"),
])
def test_edge_cases(dsa_gpu, oracle_mod, case):
    q_pos0 = case.get("q_pos0", case["N"] - case["L"])
    wl = di.Workload("edge", case["N"], case["L"], case["top_k"], 16, 17, case["kind"], q_pos0=q_pos0)
    q, k, w = di.make_indexer_inputs(wl)
    got = run_gpu(dsa_gpu, q, k, w, q_pos0, case["top_k"])
    check_rows(oracle_mod, got, q, k, w, q_pos0, case["top_k"], what=str(case))


def test_zero_queries_select_lowest_keys(dsa_gpu, oracle_mod):
    # every score is exactly 0: the selection is keys 0..k-1 (lower index wins ties);
    # these rows overflow the candidate buffer and take the blocked-fold path.
    wl = di.Workload("zero", 12000, 5, 2048, 16, 3, "zero")
    q, k, w = di.make_indexer_inputs(wl)
    got = run_gpu(dsa_gpu, q, k, w, wl.pos0, wl.top_k)
    assert np.array_equal(got, np.tile(np.arange(2048, dtype=np.int32), (5, 1)))


def _run_forced_fallback(case):
    code = (
        "import numpy as np, torch, sys\n"
        "sys.path.insert(0, '.')\n"
        "import dsa_inputs as di, dsa_sparse_attention_indexer_amd as dsa\n"
        "from tests.gpu_util import to_dev, to_dev_bf16\n"
        f"wl = di.Workload('fb', {case[0]}, {case[1]}, {case[2]}, 16, 5, '{case[3]}')\n"
        "q, k, w = di.make_indexer_inputs(wl)\n"
        "out = dsa.indexer_topk(to_dev_bf16(q), to_dev_bf16(k), to_dev(w), wl.pos0, wl.top_k)\n"
        "torch.cuda.synchronize()\n"
        "np.save(sys.argv[1], out.cpu().numpy())\n"
    )
    return code


@pytest.mark.parametrize("case", [(30000, 6, 2048, "gauss"), (20000, 4, 512, "concentrated"),
                                  (9000, 5, 256, "int"), (12000, 3, 4096, "gauss"),
                                  (6000, 4, 100, "concentrated"), (30000, 24, 2048, "gauss"),
                                  (5000, 20, 2048, "gauss"), (3000, 6, 2048, "gauss")])
def test_forced_fallback_fold_gives_same_indices(dsa_gpu, oracle_mod, tmp_path, case):
    """DSA_DEBUG_FORCE_FALLBACK=1 sends every row through the blocked fold.  The first 16 rows of
    a block are folded as up to 16 key ranges of at least top_k keys each (2 to 16 here) and
    merged, later rows (of the 24- and 20-row cases) whole; rows of fewer than 2 top_k keys (the
    3,000-key case) hold a single range and are folded whole.  The fold sorts its selection on output:
    with its 512 threads, top_k 512 .. 4,096 take the register form of the sorting network with
    1 .. 8 keys per thread, top_k 100 and 256 the LDS form."""
    wl = di.Workload("fb", case[0], case[1], case[2], 16, 5, case[3])
    q, k, w = di.make_indexer_inputs(wl)
    normal = run_gpu(dsa_gpu, q, k, w, wl.pos0, wl.top_k)
    path = tmp_path / "fb.npy"
    env = dict(os.environ, DSA_DEBUG_FORCE_FALLBACK="1")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _run_forced_fallback(case), str(path)], cwd=root, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    forced = np.load(path)
    assert np.array_equal(normal, forced)
    check_rows(oracle_mod, forced, q, k, w, wl.pos0, wl.top_k, what=f"fold {case}")


def test_run_twice_identical_and_inputs_untouched(dsa_gpu):
    import torch

    wl = di.CONFIGS["C1"]
    q, k, w = di.make_indexer_inputs(wl)
    qd, kd, wd = to_dev_bf16(q), to_dev_bf16(k), to_dev(w)
    before = [t.clone() for t in (qd, kd, wd)]
    a = dsa_gpu.indexer_topk(qd, kd, wd, wl.pos0, wl.top_k)
    b = dsa_gpu.indexer_topk(qd, kd, wd, wl.pos0, wl.top_k)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    for x, y in zip(before, (qd, kd, wd)):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


def test_causal_mask_op_matches_oracle(dsa_gpu, oracle_mod):
    import torch

    rng = np.random.default_rng(3)
    L, N, k, q_pos0 = 300, 5000, 129, 4700
    idx = rng.integers(-1, N, size=(L, k)).astype(np.int32)
    d = to_dev(idx)
    dsa_gpu.causal_mask_topk(d, q_pos0)
    torch.cuda.synchronize()
    want = oracle_mod.causal_mask(idx, q_pos0)
    assert np.array_equal(d.cpu().numpy(), want)
    dsa_gpu.causal_mask_topk(d, q_pos0)  # idempotent
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), want)
