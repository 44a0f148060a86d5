"""GPU parity of dsa_sparse_prefill against the fp64 oracle.

Tolerance (bf16 output): max |gpu - oracle| <= 2e-2 and relative L2 <= 5e-3 over
the compared tensor.  The configurations' own inputs (N(0,1)/24) give nearly
uniform attention, so the sharp-logit twin (q ~ 2 N(0,1), kv ~ N(0,1)) is also
run to exercise the softmax numerics.
"""
import numpy as np
import pytest

import dsa_inputs as di
from tests.gpu_util import assert_attn_close, bf16_dev_to_f64, report, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu
SCALE = float(np.float32(di.SOFTMAX_SCALE))


def run_gpu(dsa, q, kv, idx, q_pos0, q_block=1024, lse=True):
    import torch

    out, l = dsa.sparse_prefill(to_dev_bf16(q), to_dev_bf16(kv), to_dev(idx), q_pos0, SCALE,
                                q_block=q_block, return_lse=True)
    torch.cuda.synchronize()
    return bf16_dev_to_f64(out), l.cpu().numpy().astype(np.float64)


def check(oracle_mod, q, kv, idx, q_pos0, got, got_lse, rows=None, what=""):
    ref, ref_lse = oracle_mod.attention(q, kv, idx, q_pos0, SCALE, rows=rows)
    sub = got if rows is None else got[rows]
    sub_lse = got_lse if rows is None else got_lse[rows]
    ma, rel = assert_attn_close(sub, ref, what)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(sub_lse)), what
    assert np.max(np.abs(sub_lse[fin] - ref_lse[fin]), initial=0.0) < 1e-4, what
    report(f"{what}: max_abs={ma:.3g} rel_l2={rel:.3g}")


def attn_case(seed, L, N, H, k, q_pos0, sharp=False, minus_one=0.0, future=0.0):
    rng = np.random.default_rng(seed)
    wl = di.Workload("a", N, L, k, H, seed, "gauss", attention="sharp" if sharp else "small", q_pos0=q_pos0)
    q, kv = di.make_attention_inputs(wl, rng)
    idx = di.random_topk_indices(rng, L, N, k, q_pos0, minus_one, future)
    return q, kv, idx


def test_c0_full_with_oracle_indices(dsa_gpu, oracle_mod):
    wl = di.CONFIGS["C0"]
    inp = di.make_inputs(wl)
    idx = oracle_mod.topk(inp["q_idx"], inp["k_idx"], inp["w"], wl.pos0, wl.top_k)
    got, lse = run_gpu(dsa_gpu, inp["q"], inp["kv"], idx, wl.pos0)
    check(oracle_mod, inp["q"], inp["kv"], idx, wl.pos0, got, lse, what="C0 attention")


@pytest.mark.parametrize("H", [16, 32, 64, 128])
@pytest.mark.parametrize("sharp", [False, True])
def test_heads_and_sharp_logits(dsa_gpu, oracle_mod, H, sharp):
    q, kv, idx = attn_case(H + sharp, L=19, N=3000, H=H, k=200, q_pos0=2981, sharp=sharp)
    got, lse = run_gpu(dsa_gpu, q, kv, idx, 2981)
    check(oracle_mod, q, kv, idx, 2981, got, lse, what=f"H={H} sharp={sharp}")


def test_skips_minus_one_and_future_and_ragged_tiles(dsa_gpu, oracle_mod):
    q, kv, idx = attn_case(7, L=33, N=4000, H=64, k=77, q_pos0=3967, sharp=True, minus_one=0.2, future=0.1)
    got, lse = run_gpu(dsa_gpu, q, kv, idx, 3967)
    check(oracle_mod, q, kv, idx, 3967, got, lse, what="-1/future/ragged")


def test_short_rows_and_empty_rows(dsa_gpu, oracle_mod):
    # q_pos0 = 0: row t has t+1 causal keys; row 0 selects only key 0; a fully -1 row is empty
    q, kv, idx = attn_case(9, L=40, N=40, H=16, k=64, q_pos0=0, sharp=True)
    idx[5, :] = -1
    got, lse = run_gpu(dsa_gpu, q, kv, idx, 0)
    assert (got[5] == 0).all() and np.isneginf(lse[5]).all()
    check(oracle_mod, q, kv, idx, 0, got, lse, what="short/empty rows")


def test_single_key_copies_the_latent_row(dsa_gpu):
    q, kv, _ = attn_case(11, L=8, N=500, H=64, k=1, q_pos0=492, sharp=True)
    idx = np.arange(8, dtype=np.int32)[:, None] * 7
    got, _ = run_gpu(dsa_gpu, q, kv, idx, 492)
    lat = di.bf16_bits_to_f32(kv).astype(np.float64)[:, :512]
    for t in range(8):
        assert np.array_equal(got[t], np.broadcast_to(lat[idx[t, 0]], (64, 512)))


def test_zero_query_gives_the_mean_row(dsa_gpu, oracle_mod):
    wl = di.Workload("z", 3000, 6, 256, 64, 4, "gauss", attention="zero_q")
    q, kv = di.make_attention_inputs(wl)
    idx = di.random_topk_indices(np.random.default_rng(4), 6, 3000, 256, 2994)
    got, lse = run_gpu(dsa_gpu, q, kv, idx, 2994)
    check(oracle_mod, q, kv, idx, 2994, got, lse, what="q=0")
    assert np.allclose(lse, np.log(256.0), atol=1e-5)


@pytest.mark.parametrize("q_block", [1024, 64, 5])
def test_query_block_invariance(dsa_gpu, q_block):
    q, kv, idx = attn_case(13, L=70, N=5000, H=64, k=300, q_pos0=4930, sharp=True)
    a, la = run_gpu(dsa_gpu, q, kv, idx, 4930, q_block=70)
    b, lb = run_gpu(dsa_gpu, q, kv, idx, 4930, q_block=q_block)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_c1_full_with_gpu_indices(dsa_gpu, oracle_mod):
    wl = di.CONFIGS["C1"]
    inp = di.make_inputs(wl)
    import torch

    idx_d = dsa_gpu.indexer_topk(to_dev_bf16(inp["q_idx"]), to_dev_bf16(inp["k_idx"]), to_dev(inp["w"]),
                                 wl.pos0, wl.top_k)
    torch.cuda.synchronize()
    idx = idx_d.cpu().numpy()
    rows = np.arange(0, wl.L, 8)
    want_idx = oracle_mod.topk(inp["q_idx"], inp["k_idx"], inp["w"], wl.pos0, wl.top_k, rows=rows)
    assert np.array_equal(idx[rows], want_idx)
    got, lse = run_gpu(dsa_gpu, inp["q"], inp["kv"], idx, wl.pos0)
    check(oracle_mod, inp["q"], inp["kv"], idx, wl.pos0, got, lse, rows=rows, what="C1 attention")


@pytest.mark.parametrize("H", [16, 64])
def test_padded_kv_rows(dsa_gpu, oracle_mod, H):
    """kv rows wider than the 576 used (kv_stride 640: a latent|rope cache with padding after each
    row, passed as a column view): bit-identical to the packed rows, and the oracle agrees."""
    import torch

    q, kv, idx = attn_case(70 + H, L=23, N=2500, H=H, k=300, q_pos0=2477, sharp=True)
    wide = np.zeros((kv.shape[0], 640), np.uint16)
    wide[:, :576] = kv
    wide[:, 576:] = 0x7FC0  # NaN padding: any read of it would show
    kv_wide = to_dev_bf16(wide)[:, :576]
    assert kv_wide.stride(0) == 640
    out_w, lse_w = dsa_gpu.sparse_prefill(to_dev_bf16(q), kv_wide, to_dev(idx), 2477, SCALE, return_lse=True)
    out_p, lse_p = dsa_gpu.sparse_prefill(to_dev_bf16(q), to_dev_bf16(kv), to_dev(idx), 2477, SCALE, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out_w.view(torch.int16), out_p.view(torch.int16)), "padded rows change the output"
    assert torch.equal(lse_w, lse_p)
    check(oracle_mod, q, kv, idx, 2477, bf16_dev_to_f64(out_w), lse_w.cpu().numpy().astype(np.float64),
          what=f"kv_stride 640, H={H}")
