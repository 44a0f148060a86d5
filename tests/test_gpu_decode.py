"""GPU parity of dsa_sparse_decode (split-key attention with a log-sum-exp merge) against
the fp64 oracle, and of the decode step (indexer at L = 1, then split attention).

Same tolerance as the prefill attention: max |gpu - oracle| <= 2e-2 and relative L2 <= 5e-3
(bf16 output), lse within 1e-4.  The split result equals the unsplit kernel's up to the
rounding of the merge, so the two are compared within the same bound.
"""
import numpy as np
import pytest

import dsa_inputs as di
from tests.gpu_util import assert_attn_close, bf16_dev_to_f64, report, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu
SCALE = float(np.float32(di.SOFTMAX_SCALE))


def run_decode(dsa, q, kv, idx, q_pos0, splits=0):
    import torch

    out, l = dsa.sparse_decode(to_dev_bf16(q), to_dev_bf16(kv), to_dev(idx), q_pos0, SCALE, splits=splits,
                               return_lse=True)
    torch.cuda.synchronize()
    return bf16_dev_to_f64(out), l.cpu().numpy().astype(np.float64)


def check(oracle_mod, q, kv, idx, q_pos0, got, got_lse, what=""):
    ref, ref_lse = oracle_mod.attention(q, kv, idx, q_pos0, SCALE)
    ma, rel = assert_attn_close(got, ref, what)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(got_lse)), what
    assert np.max(np.abs(got_lse[fin] - ref_lse[fin]), initial=0.0) < 1e-4, what
    report(f"{what}: max_abs={ma:.3g} rel_l2={rel:.3g}")


def case(seed, L, N, H, k, q_pos0, sharp=True, minus_one=0.0, future=0.0):
    rng = np.random.default_rng(seed)
    wl = di.Workload("d", N, L, k, H, seed, "gauss", attention="sharp" if sharp else "small", q_pos0=q_pos0)
    q, kv = di.make_attention_inputs(wl, rng)
    idx = di.random_topk_indices(rng, L, N, k, q_pos0, minus_one, future)
    return q, kv, idx


@pytest.mark.parametrize("splits", [0, 1, 3, 16, 128])
def test_decode_splits(dsa_gpu, oracle_mod, splits):
    q, kv, idx = case(100 + splits, L=1, N=3000, H=64, k=512, q_pos0=2999)
    got, lse = run_decode(dsa_gpu, q, kv, idx, 2999, splits)
    check(oracle_mod, q, kv, idx, 2999, got, lse, what=f"decode splits={splits}")


@pytest.mark.parametrize("H", [16, 32, 128])
@pytest.mark.parametrize("sharp", [False, True])
def test_decode_heads(dsa_gpu, oracle_mod, H, sharp):
    q, kv, idx = case(200 + H + sharp, L=1, N=2500, H=H, k=300, q_pos0=2499, sharp=sharp)
    got, lse = run_decode(dsa_gpu, q, kv, idx, 2499)
    check(oracle_mod, q, kv, idx, 2499, got, lse, what=f"decode H={H} sharp={sharp}")


def test_short_chunk_with_minus_one_future_and_ragged_tail(dsa_gpu, oracle_mod):
    q, kv, idx = case(301, L=5, N=4000, H=64, k=77, q_pos0=3995, minus_one=0.3, future=0.1)
    got, lse = run_decode(dsa_gpu, q, kv, idx, 3995, splits=3)
    check(oracle_mod, q, kv, idx, 3995, got, lse, what="short chunk, -1/future/ragged")


def test_empty_splits_and_empty_rows(dsa_gpu, oracle_mod):
    # q_pos0 = 0: row t has t + 1 causal keys, so most of each list is -1 and later splits
    # are empty; row 3 is -1 throughout (output 0, lse -inf).
    q, kv, idx = case(302, L=6, N=6, H=16, k=96, q_pos0=0)
    idx[3, :] = -1
    got, lse = run_decode(dsa_gpu, q, kv, idx, 0, splits=3)
    assert (got[3] == 0).all() and np.isneginf(lse[3]).all()
    check(oracle_mod, q, kv, idx, 0, got, lse, what="empty splits/rows")


def test_decode_equals_prefill(dsa_gpu):
    import torch

    q, kv, idx = case(303, L=3, N=6000, H=64, k=1000, q_pos0=5997)
    qd, kvd, idd = to_dev_bf16(q), to_dev_bf16(kv), to_dev(idx)
    a, la = dsa_gpu.sparse_prefill(qd, kvd, idd, 5997, SCALE, return_lse=True)
    b, lb = dsa_gpu.sparse_decode(qd, kvd, idd, 5997, SCALE, splits=7, return_lse=True)
    torch.cuda.synchronize()
    ma, rel = assert_attn_close(bf16_dev_to_f64(b), bf16_dev_to_f64(a), "decode vs prefill")
    assert torch.allclose(la, lb, atol=1e-5, rtol=0)
    report(f"decode vs prefill: max_abs={ma:.3g} rel_l2={rel:.3g}")


def test_c3_decode_step(dsa_gpu, oracle_mod):
    """The decode step at the headline cache size: the newest position's query selects its
    top 2,048 of 131,072 keys (indexer at L = 1), then the split attention runs over them."""
    import torch

    wl = di.CONFIGS["C3"]
    inp = di.make_inputs(wl)
    t = wl.L - 1  # the newest query of the chunk sits at position N - 1
    q_idx, w, q = inp["q_idx"][t:t + 1], inp["w"][t:t + 1], inp["q"][t:t + 1]
    pos = wl.pos0 + t
    idx_d = dsa_gpu.indexer_topk(to_dev_bf16(q_idx), to_dev_bf16(inp["k_idx"]), to_dev(w), pos, wl.top_k)
    torch.cuda.synchronize()
    idx = idx_d.cpu().numpy()
    want = oracle_mod.topk(q_idx, inp["k_idx"], w, pos, wl.top_k)
    assert np.array_equal(idx, want)
    got, lse = run_decode(dsa_gpu, q, inp["kv"], idx, pos)
    check(oracle_mod, q, inp["kv"], idx, pos, got, lse, what="C3 decode step")
