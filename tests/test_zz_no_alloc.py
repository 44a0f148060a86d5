"""dsa_indexer_topk_noalloc, the indexer entry point that takes no workspace (its scratch is
a static device array in the library), against dsa_indexer_topk with a caller workspace.
Both are called through the C ABI; the indices must agree bit for bit, on two calls in a
row, the second smaller than the first (the scratch keeps the first call's contents)."""
import ctypes

import numpy as np
import pytest

import dsa_inputs as di
from tests.gpu_util import report, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def run(lib, noalloc, q, k, w, pos0, top_k, q_block):
    import torch

    L, nh, hd = q.shape
    N = k.shape[0]
    out = torch.full((L, top_k), -7, dtype=torch.int32, device=q.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        st = lib.dsa_indexer_topk_noalloc(q.data_ptr(), k.data_ptr(), w.data_ptr(), L, N, nh, hd, pos0, top_k,
                                          q_block, out.data_ptr(), stream)
    else:
        need = lib.dsa_indexer_topk_workspace_bytes(L, N, top_k, q_block)
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        st = lib.dsa_indexer_topk(q.data_ptr(), k.data_ptr(), w.data_ptr(), L, N, nh, hd, pos0, top_k, q_block,
                                  out.data_ptr(), ws.data_ptr(), need, stream)
    assert st == 0, lib.dsa_last_error()
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_noalloc_matches_the_workspace_entry_point(dsa_gpu):
    lib = dsa_gpu.load_library()
    cases = [
        di.Workload("na1", 16384, 512, 2048, 16, 1, "gauss"),          # 48 MiB of scratch
        di.Workload("na2", 9000, 37, 512, 16, 2, "concentrated"),      # smaller, ragged group
    ]
    for wl in cases:
        q, k, w = (to_dev_bf16(x) if x.dtype == np.uint16 else to_dev(x) for x in di.make_indexer_inputs(wl))
        need = lib.dsa_indexer_topk_workspace_bytes(wl.L, wl.N, wl.top_k, 0)
        assert 0 < need <= dsa_gpu.NOALLOC_SCRATCH_BYTES
        ref = run(lib, False, q, k, w, wl.pos0, wl.top_k, 0)
        got = run(lib, True, q, k, w, wl.pos0, wl.top_k, 0)
        assert (ref >= 0).all()
        assert np.array_equal(got, ref), f"{wl.name}: no-allocation indices differ"
        report(f"{wl.name}: L={wl.L} N={wl.N} top_k={wl.top_k}: identical ({need / 2**20:.1f} MiB of scratch)")


def test_noalloc_rejects_sizes_above_its_scratch(dsa_gpu):
    import torch

    lib = dsa_gpu.load_library()
    wl = di.Workload("big", 131072, 2048, 2048, 16, 3, "gauss")
    assert lib.dsa_indexer_topk_workspace_bytes(wl.L, wl.N, wl.top_k, 1024) > dsa_gpu.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((wl.L, 32, 128), dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros((wl.N, 128), dtype=torch.bfloat16, device="cuda:0")
    w = torch.zeros((wl.L, 32), dtype=torch.float32, device="cuda:0")
    out = torch.full((wl.L, wl.top_k), -7, dtype=torch.int32, device="cuda:0")
    st = lib.dsa_indexer_topk_noalloc(q.data_ptr(), k.data_ptr(), w.data_ptr(), wl.L, wl.N, 32, 128, wl.pos0,
                                      wl.top_k, 1024, out.data_ptr(), None)
    assert st == 3 and b"static scratch" in lib.dsa_last_error()
    torch.cuda.synchronize()
    assert (out == -7).all()  # nothing written
