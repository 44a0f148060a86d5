"""The append-only indexer key cache (dsa_indexer_key_cache_*, dsa_indexer_topk_cached)
against dsa_indexer_topk, which lays out every key on each call: indices bit for bit,
and the selection counters (which depend on the error bound from the key statistics)
equal, as the cache grows by chunks of many keys and by single keys (decode), across a
restart, and at the 128K-key cache of a decode step against the oracle."""
import numpy as np
import pytest

import dsa_inputs as di
from tests.gpu_util import report, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def both(dsa, q, k, w, pos0, top_k, cache):
    import torch

    L, N = q.shape[0], k.shape[0]
    ws_a = torch.empty(dsa.workspace_bytes(L, N, top_k), dtype=torch.uint8, device="cuda:0")
    ws_b = torch.empty(dsa.cached_workspace_bytes(L, N, top_k), dtype=torch.uint8, device="cuda:0")
    a = dsa.indexer_topk(q, k, w, pos0, top_k, workspace=ws_a)
    b = dsa.indexer_topk_cached(q, k, w, pos0, top_k, cache, workspace=ws_b)
    sa, sb = dsa.indexer_stats(ws_a), dsa.indexer_stats(ws_b)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy(), sa, sb


def test_growing_cache_matches_full_layout(dsa_gpu):
    wl = di.Workload("kc", 40000, 64, 2048, 16, 61, "concentrated")
    q, k, w = di.make_indexer_inputs(wl)
    kd = to_dev_bf16(k)
    cache = dsa_gpu.KeyCache(wl.N)
    checked = 0
    for n in [30000, 30001, 30002, 30009, 30040, 31000, 39999, 40000]:
        cache.append(kd, n)
        for L in (1, 64):
            t0 = n - L  # the newest L positions of the n keys appended so far
            qd, wd = to_dev_bf16(q[:L]), to_dev(w[:L])
            a, b, sa, sb = both(dsa_gpu, qd, kd[:n], wd, t0, wl.top_k, cache)
            assert np.array_equal(a, b), f"n={n} L={L}: cached indices differ"
            assert sa == sb, f"n={n} L={L}: selection counters differ: {sa} vs {sb}"
            checked += 1
    report(f"key cache grown 30000 -> 40000: {checked} calls identical to the full layout")


def test_restart_resets_the_statistics(dsa_gpu):
    """Keys 64x larger first; after a restart (n_old = 0) the cache's statistics must be those
    of the new keys alone, or the error bound, and with it the fp64 band, would be 64x wider."""
    wl = di.Workload("kr", 20000, 16, 1024, 16, 62, "gauss")
    q, k, w = di.make_indexer_inputs(wl)
    big = di.f32_to_bf16_bits(di.bf16_bits_to_f32(k) * np.float32(64.0))
    cache = dsa_gpu.KeyCache(wl.N)
    cache.append(to_dev_bf16(big))
    cache.reset()
    kd = to_dev_bf16(k)
    cache.append(kd)
    a, b, sa, sb = both(dsa_gpu, to_dev_bf16(q), kd, to_dev(w), wl.pos0, wl.top_k, cache)
    assert np.array_equal(a, b) and sa == sb, f"{sa} vs {sb}"


def test_decode_at_128k_against_the_oracle(dsa_gpu, oracle_mod):
    wl = di.CONFIGS["C3"]
    q, k, w = di.make_indexer_inputs(wl)
    kd = to_dev_bf16(k)
    cache = dsa_gpu.KeyCache(wl.N)
    cache.append(kd, wl.N - 1)
    cache.append(kd)  # the decode step appends the newest key
    t = wl.L - 1
    got = dsa_gpu.indexer_topk_cached(to_dev_bf16(q[t:t + 1]), kd, to_dev(w[t:t + 1]), wl.pos0 + t, wl.top_k, cache)
    want = oracle_mod.topk(q[t:t + 1], k, w[t:t + 1], wl.pos0 + t, wl.top_k)
    assert np.array_equal(got.cpu().numpy(), want)
