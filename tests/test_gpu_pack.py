"""GPU parity of dsa_sparse_prefill_packed (LiteDSA neighbour packing: query pairs attend
over the union of their index rows, each masking the keys it did not select) against the
fp64 oracle, at the prefill attention's tolerance (max-abs 2e-2, rel-L2 5e-3, lse 1e-4).

Index rows come with a chosen overlap between neighbours (0 = independent, 0.9 = each row
keeps about 90% of the previous row's keys), ascending with a -1 tail as the indexer writes
them (merged union), or scrambled / with -1 holes / with future keys (concatenated union).
"""
import numpy as np
import pytest

import dsa_inputs as di
from tests.gpu_util import assert_attn_close, bf16_dev_to_f64, report, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu
SCALE = float(np.float32(di.SOFTMAX_SCALE))


def inputs(seed, L, N, H, k, q_pos0, keep):
    rng = np.random.default_rng(seed)
    wl = di.Workload("p", N, L, k, H, seed, "gauss", attention="sharp", q_pos0=q_pos0)
    q, kv = di.make_attention_inputs(wl, rng)
    idx = di.overlapping_topk_indices(rng, L, N, k, q_pos0, keep)
    return q, kv, idx


def run(dsa, q, kv, idx, q_pos0, pack=True, q_block=1024):
    import torch

    out, lse = dsa.sparse_prefill(to_dev_bf16(q), to_dev_bf16(kv), to_dev(idx), q_pos0, SCALE, q_block=q_block,
                                  return_lse=True, pack=pack)
    torch.cuda.synchronize()
    return bf16_dev_to_f64(out), lse.cpu().numpy().astype(np.float64)


def check(oracle_mod, q, kv, idx, q_pos0, got, got_lse, what):
    ref, ref_lse = oracle_mod.attention(q, kv, idx, q_pos0, SCALE)
    ma, rel = assert_attn_close(got, ref, what)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(got_lse)), what
    assert np.max(np.abs(got_lse[fin] - ref_lse[fin]), initial=0.0) < 1e-4, what
    report(f"{what}: max_abs={ma:.3g} rel_l2={rel:.3g}")


@pytest.mark.parametrize("keep", [0.0, 0.5, 0.9, 1.0])
def test_overlap_levels(dsa_gpu, oracle_mod, keep):
    """37 queries (an odd count: the last pair has one query), top_k 300 (a ragged last tile)."""
    q, kv, idx = inputs(10, L=37, N=4000, H=64, k=300, q_pos0=3963, keep=keep)
    got, lse = run(dsa_gpu, q, kv, idx, 3963)
    check(oracle_mod, q, kv, idx, 3963, got, lse, f"packed keep={keep}")


@pytest.mark.parametrize("H", [16, 32])
def test_fewer_heads(dsa_gpu, oracle_mod, H):
    q, kv, idx = inputs(11 + H, L=20, N=3000, H=H, k=256, q_pos0=2980, keep=0.8)
    got, lse = run(dsa_gpu, q, kv, idx, 2980)
    check(oracle_mod, q, kv, idx, 2980, got, lse, f"packed H={H}")


def test_unsorted_rows_holes_and_future_keys(dsa_gpu, oracle_mod):
    """Rows that are not ascending-with-a-tail take the concatenated union; future keys and
    -1 anywhere are skipped per query."""
    rng = np.random.default_rng(12)
    q, kv, idx = inputs(12, L=16, N=5000, H=64, k=200, q_pos0=4000, keep=0.7)
    idx[3] = idx[3][rng.permutation(200)]               # scrambled
    idx[5, 17] = -1                                     # a hole
    idx[8, -5:] = rng.integers(4010, 5000, size=5)      # future keys for query 8 (position 4008)
    got, lse = run(dsa_gpu, q, kv, idx, 4000)
    check(oracle_mod, q, kv, idx, 4000, got, lse, "packed unsorted/holes/future")


def test_early_positions_with_minus_one_tails(dsa_gpu, oracle_mod):
    """q_pos0 = 0: row t has t + 1 causal keys, so most of every row is the -1 tail."""
    q, kv, idx = inputs(13, L=40, N=40, H=32, k=64, q_pos0=0, keep=0.9)
    got, lse = run(dsa_gpu, q, kv, idx, 0)
    check(oracle_mod, q, kv, idx, 0, got, lse, "packed early positions")


def test_odd_query_blocks_and_unpacked_fallbacks(dsa_gpu, oracle_mod):
    """q_block 5 leaves single queries at block ends; H = 128 and top_k > 2048 run unpacked."""
    q, kv, idx = inputs(14, L=23, N=6000, H=64, k=500, q_pos0=5977, keep=0.8)
    got, lse = run(dsa_gpu, q, kv, idx, 5977, q_block=5)
    check(oracle_mod, q, kv, idx, 5977, got, lse, "packed q_block=5")
    q, kv, idx = inputs(15, L=6, N=3000, H=128, k=100, q_pos0=2994, keep=0.8)
    got, lse = run(dsa_gpu, q, kv, idx, 2994)
    check(oracle_mod, q, kv, idx, 2994, got, lse, "H=128 (unpacked)")
    q, kv, idx = inputs(16, L=4, N=5000, H=16, k=2100, q_pos0=4996, keep=0.8)
    got, lse = run(dsa_gpu, q, kv, idx, 4996)
    check(oracle_mod, q, kv, idx, 4996, got, lse, "top_k=2100 (unpacked)")


def test_packed_matches_unpacked(dsa_gpu):
    from tests.gpu_util import attn_errors

    q, kv, idx = inputs(17, L=64, N=20000, H=64, k=2048, q_pos0=19936, keep=0.85)
    a, la = run(dsa_gpu, q, kv, idx, 19936, pack=True)
    b, lb = run(dsa_gpu, q, kv, idx, 19936, pack=False)
    ma, rel = attn_errors(a, b)
    assert ma <= 2e-2 and rel <= 5e-3
    assert np.max(np.abs(la - lb)) < 1e-4


def test_indexer_then_packed_attention(dsa_gpu, oracle_mod):
    """The indexer's own output (ascending, -1 tail) feeds the packed attention."""
    import torch

    wl = di.Workload("pk", 6000, 48, 512, 64, 18, "gauss", attention="small")
    inp = di.make_inputs(wl)
    idx = dsa_gpu.indexer_topk(to_dev_bf16(inp["q_idx"]), to_dev_bf16(inp["k_idx"]), to_dev(inp["w"]), wl.pos0,
                               wl.top_k)
    out, lse = dsa_gpu.sparse_prefill(to_dev_bf16(inp["q"]), to_dev_bf16(inp["kv"]), idx, wl.pos0, SCALE,
                                      return_lse=True, pack=True)
    torch.cuda.synchronize()
    check(oracle_mod, inp["q"], inp["kv"], idx.cpu().numpy(), wl.pos0, bf16_dev_to_f64(out),
          lse.cpu().numpy().astype(np.float64), "indexer -> packed")
