"""The library's calls are capturable in a HIP graph (they enqueue kernels only: no host
synchronisation, no allocation, no memset nodes).  Each test captures a path once, replays it
several times with eager work and synchronisations in between, and requires every replay to
equal the eager result bit for bit (the kernels are deterministic)."""
import numpy as np
import pytest

import dsa_inputs as di
from tests.gpu_util import to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu
SCALE = float(np.float32(di.SOFTMAX_SCALE))


def capture(fn):
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up on the side stream, as torch recommends before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_prefill_step_graph_replays_match_eager(dsa_gpu):
    import torch

    wl = di.CONFIGS["C1"]
    inp = di.make_inputs(wl)
    q_idx, k_idx, w = to_dev_bf16(inp["q_idx"]), to_dev_bf16(inp["k_idx"]), to_dev(inp["w"])
    q, kv = to_dev_bf16(inp["q"]), to_dev_bf16(inp["kv"])
    idx = torch.empty((wl.L, wl.top_k), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.L, wl.H, 512), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(dsa_gpu.workspace_bytes(wl.L, wl.N, wl.top_k, 256), dtype=torch.uint8, device="cuda")

    def step():
        dsa_gpu.indexer_topk(q_idx, k_idx, w, wl.pos0, wl.top_k, q_block=256, out=idx, workspace=ws)
        dsa_gpu.sparse_prefill(q, kv, idx, wl.pos0, SCALE, q_block=256, out=out)

    step()
    torch.cuda.synchronize()
    ref_idx, ref_out = idx.clone(), out.clone()
    g = capture(step)
    for rep in range(4):
        idx.fill_(-7)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), f"replay {rep}: indices"
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"replay {rep}: output"
        step()  # eager work between replays
        torch.cuda.synchronize()


def test_decode_step_and_batch_graph_replays_match_eager(dsa_gpu):
    import torch

    rng = np.random.default_rng(5)
    wl = di.Workload("g", 20000, 1, 2048, 64, 6, "gauss", attention="sharp", q_pos0=19999)
    inp = di.make_inputs(wl)
    q_idx, k_idx, w = to_dev_bf16(inp["q_idx"]), to_dev_bf16(inp["k_idx"]), to_dev(inp["w"])
    q, kv = to_dev_bf16(inp["q"]), to_dev_bf16(inp["kv"])
    idx = torch.empty((1, 2048), dtype=torch.int32, device="cuda")
    out = torch.empty((1, 64, 512), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(dsa_gpu.workspace_bytes(1, wl.N, 2048, 0), dtype=torch.uint8, device="cuda")
    dws = torch.empty(dsa_gpu.decode_workspace_bytes(1, 64, 2048), dtype=torch.uint8, device="cuda")
    # a batch of three sequences through the varlen calls (their tables are written by kernels)
    cu_q, cu_k, pos0 = [0, 1, 3, 4], [0, 7000, 12000, 20000], [6999, 4998, 7999]
    bq = to_dev_bf16(inp["q_idx"].repeat(4, axis=0))
    bw = to_dev(np.ascontiguousarray(inp["w"].repeat(4, axis=0)))
    bidx = torch.empty((4, 2048), dtype=torch.int32, device="cuda")
    bws = torch.empty(dsa_gpu.varlen_workspace_bytes(cu_q, cu_k, pos0, 2048), dtype=torch.uint8, device="cuda")

    def step():
        dsa_gpu.indexer_topk(q_idx, k_idx, w, 19999, 2048, out=idx, workspace=ws)
        dsa_gpu.sparse_decode(q, kv, idx, 19999, SCALE, out=out, workspace=dws)
        dsa_gpu.indexer_topk_varlen(bq, k_idx, bw, cu_q, cu_k, pos0, 2048, out=bidx, workspace=bws)

    step()
    torch.cuda.synchronize()
    ref = (idx.clone(), out.clone(), bidx.clone())
    g = capture(step)
    for rep in range(4):
        idx.fill_(-7)
        bidx.fill_(-7)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]) and torch.equal(bidx, ref[2]), f"replay {rep}: indices"
        assert torch.equal(out.view(torch.int16), ref[1].view(torch.int16)), f"replay {rep}: output"
        step()
        torch.cuda.synchronize()
