"""GPU parity of the batched (varlen) entry points: dsa_indexer_topk_varlen and
dsa_sparse_prefill_varlen.

A batch packs sequences of different lengths, cache sizes and start positions.  Each
sequence's rows must equal the oracle on that sequence alone (indices bit-exact,
attention within the prefill tolerance), and must be bit-identical to the one-sequence
entry point on it: batching only changes where rows live, not what a row computes.
"""
import numpy as np
import pytest

import dsa_inputs as di
from tests.gpu_util import assert_attn_close, bf16_dev_to_f64, bits_of, report, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu
SCALE = float(np.float32(di.SOFTMAX_SCALE))


def make_batch(specs, top_k, H=64, seed=0, attention="sharp"):
    """specs: (N, L, pos0, indexer kind) per sequence -> per-sequence inputs and the packed batch."""
    seqs = []
    for i, (N, L, p0, kind) in enumerate(specs):
        wl = di.Workload(f"s{i}", N, L, top_k, H, 1000 * seed + i, kind, attention=attention, q_pos0=p0)
        rng = di.make_rng(wl.seed)
        q_idx, k_idx, w = di.make_indexer_inputs(wl, rng)
        q, kv = di.make_attention_inputs(wl, rng)
        seqs.append(dict(wl=wl, q_idx=q_idx, k_idx=k_idx, w=w, q=q, kv=kv))
    cu_q = np.cumsum([0] + [s["wl"].L for s in seqs]).astype(np.int64)
    cu_k = np.cumsum([0] + [s["wl"].N for s in seqs]).astype(np.int64)
    pos0 = np.array([s["wl"].pos0 for s in seqs], dtype=np.int64)
    cat = lambda key, shape: (np.concatenate([s[key] for s in seqs]) if seqs else np.zeros(shape))
    packed = dict(q_idx=cat("q_idx", (0, 32, 128)).astype(np.uint16), k_idx=cat("k_idx", (0, 128)).astype(np.uint16),
                  w=cat("w", (0, 32)).astype(np.float32), q=cat("q", (0, H, 576)).astype(np.uint16),
                  kv=cat("kv", (0, 576)).astype(np.uint16))
    return seqs, cu_q, cu_k, pos0, packed


def run_indexer_varlen(dsa, packed, cu_q, cu_k, pos0, top_k, q_block=1024):
    import torch

    kd = to_dev_bf16(packed["k_idx"]) if packed["k_idx"].shape[0] else torch.zeros((1, 128), dtype=torch.bfloat16,
                                                                                   device="cuda:0")
    out = dsa.indexer_topk_varlen(to_dev_bf16(packed["q_idx"]), kd, to_dev(packed["w"]), cu_q, cu_k, pos0, top_k,
                                  q_block=q_block)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_indexer(oracle_mod, seqs, cu_q, got, top_k, what):
    for b, s in enumerate(seqs):
        wl = s["wl"]
        if wl.L == 0:
            continue
        want = oracle_mod.topk(s["q_idx"], s["k_idx"], s["w"], wl.pos0, top_k)
        sub = got[cu_q[b]:cu_q[b + 1]]
        bad = np.nonzero((sub != want).any(axis=1))[0]
        assert bad.size == 0, f"{what}: sequence {b} ({wl.N} keys, {wl.L} rows): {bad.size} rows differ"
    report(f"{what}: {len(seqs)} sequences, {int(cu_q[-1])} rows bit-exact")


RAGGED = [(5000, 70, 100, "gauss"), (20000, 1, 19999, "gauss"), (2000, 300, 1700, "gauss"),
          (9000, 37, 8963, "sink"), (700, 9, 3, "int")]


@pytest.mark.parametrize("top_k", [256, 2048])
def test_ragged_batch_matches_oracle(dsa_gpu, oracle_mod, top_k):
    seqs, cu_q, cu_k, pos0, packed = make_batch(RAGGED, top_k, seed=1)
    got = run_indexer_varlen(dsa_gpu, packed, cu_q, cu_k, pos0, top_k)
    check_indexer(oracle_mod, seqs, cu_q, got, top_k, f"ragged top_k={top_k}")


@pytest.mark.parametrize("q_block", [8, 24, 100, 1024])
def test_batch_equals_single_sequence_calls(dsa_gpu, q_block):
    """Blocks of 8..1024 rows: sequences straddle blocks and blocks hold several sequences."""
    import torch

    top_k = 256
    seqs, cu_q, cu_k, pos0, packed = make_batch(RAGGED, top_k, seed=2)
    got = run_indexer_varlen(dsa_gpu, packed, cu_q, cu_k, pos0, top_k, q_block)
    for b, s in enumerate(seqs):
        wl = s["wl"]
        one = dsa_gpu.indexer_topk(to_dev_bf16(s["q_idx"]), to_dev_bf16(s["k_idx"]), to_dev(s["w"]), wl.pos0, top_k)
        torch.cuda.synchronize()
        assert np.array_equal(got[cu_q[b]:cu_q[b + 1]], one.cpu().numpy()), f"sequence {b}, q_block={q_block}"


def test_decode_batch_matches_oracle(dsa_gpu, oracle_mod):
    """48 sequences of one query each (a decode step over a batch), caches of 1 .. 30,000 keys."""
    rng = np.random.default_rng(7)
    Ns = np.concatenate([[1, 2, 255, 256, 257, 2048, 2049], rng.integers(1, 30000, size=41)])
    specs = [(int(n), 1, int(n) - 1, "gauss" if i % 3 else "concentrated") for i, n in enumerate(Ns)]
    top_k = 2048
    seqs, cu_q, cu_k, pos0, packed = make_batch(specs, top_k, seed=3)
    got = run_indexer_varlen(dsa_gpu, packed, cu_q, cu_k, pos0, top_k)
    check_indexer(oracle_mod, seqs, cu_q, got, top_k, "decode batch")


def test_empty_sequences_and_empty_batch(dsa_gpu, oracle_mod):
    import torch

    specs = [(0, 0, 0, "gauss"), (4000, 0, 10, "gauss"), (4000, 17, 3983, "gauss"), (0, 0, 0, "gauss"),
             (1, 1, 0, "gauss"), (6000, 0, 0, "gauss")]
    top_k = 512
    seqs, cu_q, cu_k, pos0, packed = make_batch(specs, top_k, seed=4)
    got = run_indexer_varlen(dsa_gpu, packed, cu_q, cu_k, pos0, top_k)
    assert got.shape == (18, top_k)
    check_indexer(oracle_mod, seqs, cu_q, got, top_k, "empty sequences")
    # no query rows at all: a no-op that leaves the output untouched
    out = torch.full((0, top_k), 7, dtype=torch.int32, device="cuda:0")
    q0 = torch.zeros((0, 32, 128), dtype=torch.bfloat16, device="cuda:0")
    k0 = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda:0")
    w0 = torch.zeros((0, 32), dtype=torch.float32, device="cuda:0")
    dsa_gpu.indexer_topk_varlen(q0, k0, w0, [0, 0, 0], [0, 4, 8], [0, 2], top_k, out=out)
    dsa_gpu.indexer_topk_varlen(q0, k0, w0, [0], [0], [], top_k, out=out)
    torch.cuda.synchronize()


def test_many_sequences_fill_several_table_chunks(dsa_gpu, oracle_mod):
    """70 sequences: the tables are written 32 sequences per launch."""
    rng = np.random.default_rng(11)
    specs = []
    for i in range(70):
        N = int(rng.integers(1, 3000))
        L = int(rng.integers(0, min(N, 20) + 1))
        specs.append((N, L, int(rng.integers(0, N - L + 1)), "gauss"))
    top_k = 128
    seqs, cu_q, cu_k, pos0, packed = make_batch(specs, top_k, seed=5)
    got = run_indexer_varlen(dsa_gpu, packed, cu_q, cu_k, pos0, top_k, q_block=64)
    check_indexer(oracle_mod, seqs, cu_q, got, top_k, "70 sequences")


def test_forced_fallback_fold_on_a_batch(dsa_gpu, oracle_mod, monkeypatch):
    """DSA_DEBUG_FORCE_FALLBACK=1 sends every scored row of the batch through the blocked fold."""
    top_k = 256
    seqs, cu_q, cu_k, pos0, packed = make_batch(RAGGED, top_k, seed=6)
    normal = run_indexer_varlen(dsa_gpu, packed, cu_q, cu_k, pos0, top_k)
    monkeypatch.setenv("DSA_DEBUG_FORCE_FALLBACK", "1")
    forced = run_indexer_varlen(dsa_gpu, packed, cu_q, cu_k, pos0, top_k)
    monkeypatch.delenv("DSA_DEBUG_FORCE_FALLBACK")
    assert np.array_equal(normal, forced)
    check_indexer(oracle_mod, seqs, cu_q, forced, top_k, "batch fold")


# ------------------------------------------------------------------ attention

def run_attn_varlen(dsa, packed, idx, cu_q, cu_k, pos0, splits):
    import torch

    out, lse = dsa.sparse_prefill_varlen(to_dev_bf16(packed["q"]), to_dev_bf16(packed["kv"]), to_dev(idx), cu_q,
                                         cu_k, pos0, SCALE, splits=splits, return_lse=True)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("splits", [1, 0, 4])
def test_attention_batch_matches_oracle(dsa_gpu, oracle_mod, splits):
    top_k = 300
    specs = [(5000, 70, 100, "gauss"), (20000, 1, 19999, "gauss"), (3000, 513, 2487, "gauss"), (40, 5, 0, "gauss")]
    seqs, cu_q, cu_k, pos0, packed = make_batch(specs, top_k, H=32, seed=7)
    rng = np.random.default_rng(8)
    idx = np.concatenate([di.random_topk_indices(rng, s["wl"].L, s["wl"].N, top_k, s["wl"].pos0, 0.1, 0.1)
                          for s in seqs])
    out, lse = run_attn_varlen(dsa_gpu, packed, idx, cu_q, cu_k, pos0, splits)
    got, got_lse = bf16_dev_to_f64(out), lse.cpu().numpy().astype(np.float64)
    for b, s in enumerate(seqs):
        wl = s["wl"]
        sl = slice(cu_q[b], cu_q[b + 1])
        ref, ref_lse = oracle_mod.attention(s["q"], s["kv"], idx[sl], wl.pos0, SCALE)
        assert_attn_close(got[sl], ref, f"sequence {b} splits={splits}")
        fin = np.isfinite(ref_lse)
        assert np.array_equal(fin, np.isfinite(got_lse[sl]))
        assert np.max(np.abs(got_lse[sl][fin] - ref_lse[fin]), initial=0.0) < 1e-4
    report(f"attention batch splits={splits}: {len(seqs)} sequences within tolerance")


def test_attention_batch_equals_single_sequence_calls(dsa_gpu):
    """splits = 1 runs the prefill kernel on each row exactly as the one-sequence call does."""
    import torch

    top_k = 512
    seqs, cu_q, cu_k, pos0, packed = make_batch(RAGGED[:4], top_k, H=64, seed=9)
    rng = np.random.default_rng(10)
    idx = np.concatenate([di.random_topk_indices(rng, s["wl"].L, s["wl"].N, top_k, s["wl"].pos0)
                          for s in seqs])
    out, lse = run_attn_varlen(dsa_gpu, packed, idx, cu_q, cu_k, pos0, 1)
    for b, s in enumerate(seqs):
        sl = slice(cu_q[b], cu_q[b + 1])
        o1, l1 = dsa_gpu.sparse_prefill(to_dev_bf16(s["q"]), to_dev_bf16(s["kv"]), to_dev(idx[sl]), s["wl"].pos0,
                                        SCALE, return_lse=True)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(out[sl]), bits_of(o1)), f"sequence {b}"
        assert torch.equal(lse[sl], l1)


def test_indexer_then_attention_on_a_batch(dsa_gpu, oracle_mod):
    """The whole path on a batch: packed indexer output feeds the packed attention."""
    import torch

    top_k = 256
    specs = [(4000, 33, 3967, "gauss"), (900, 1, 899, "gauss"), (2500, 130, 0, "concentrated")]
    seqs, cu_q, cu_k, pos0, packed = make_batch(specs, top_k, H=16, seed=12)
    idx = dsa_gpu.indexer_topk_varlen(to_dev_bf16(packed["q_idx"]), to_dev_bf16(packed["k_idx"]),
                                      to_dev(packed["w"]), cu_q, cu_k, pos0, top_k)
    out = dsa_gpu.sparse_prefill_varlen(to_dev_bf16(packed["q"]), to_dev_bf16(packed["kv"]), idx, cu_q, cu_k, pos0,
                                        SCALE)
    torch.cuda.synchronize()
    got_idx, got = idx.cpu().numpy(), bf16_dev_to_f64(out)
    check_indexer(oracle_mod, seqs, cu_q, got_idx, top_k, "path indexer")
    for b, s in enumerate(seqs):
        sl = slice(cu_q[b], cu_q[b + 1])
        ref, _ = oracle_mod.attention(s["q"], s["kv"], got_idx[sl], s["wl"].pos0, SCALE)
        assert_attn_close(got[sl], ref, f"path sequence {b}")
