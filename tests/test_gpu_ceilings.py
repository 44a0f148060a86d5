"""The measured-ceiling kernels (dsa_ceiling_mfma_bf16, dsa_ceiling_stream) that bench.py reports
beside the published peaks: they must do the work they are timed for.

- With constant operands (every bf16 operand 1.0) each MFMA adds 16 to each of its 16 accumulator
  elements per lane, so after iters x 8 MFMAs a thread's sum is 8 * 16 * 16 * iters exactly.
- With random operands the sums are finite and not all equal.
- The copy reproduces its source bit for bit; the read-only stream reads every element: each
  workgroup streams one contiguous chunk (a whole number of 2,048-element tiles, the last chunk
  ragged), so thread t of workgroup b XORs the words of the chunk's elements t, t + 256, ...
"""
import numpy as np
import pytest

from tests.gpu_util import report

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wps", [1, 2])
def test_mfma_ceiling_does_its_work(dsa_gpu, wps):
    import torch

    n = dsa_gpu.ceiling_mfma_threads(wps)
    assert n >= 256 * wps
    out = torch.full((n,), -1.0, dtype=torch.float32, device="cuda:0")
    iters = 37
    flops = dsa_gpu.ceiling_mfma(out, iters, False, wps)
    torch.cuda.synchronize()
    assert flops == (n // 64) * iters * 8 * 32768
    assert (out.cpu().numpy() == 8 * 16 * 16 * iters).all()
    dsa_gpu.ceiling_mfma(out, iters, True, wps)
    torch.cuda.synchronize()
    v = out.cpu().numpy()
    assert np.isfinite(v).all() and np.unique(v).size > n // 2
    report(f"mfma ceiling ({wps} wave/SIMD): {n} threads checked")


def test_stream_ceiling_copies_and_reads(dsa_gpu):
    import torch

    n = 2048 * 1024 + 777  # 16-byte elements: full chunks, a ragged one, then idle workgroups
    g = torch.Generator(device="cpu").manual_seed(7)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (4 * n,), dtype=torch.int32, generator=g).to("cuda:0")
    for nt in (False, True):
        dst = torch.zeros_like(src)
        dsa_gpu.ceiling_stream(src, dst, nontemporal=nt)
        torch.cuda.synchronize()
        assert torch.equal(src, dst)
    words = dsa_gpu.ceiling_stream_sink_words()
    blocks, tile = words // 256, 8 * 256
    per = -(-n // (blocks * tile)) * tile
    host = src.cpu().numpy().view(np.uint32)
    pad = np.zeros(blocks * per * 4, np.uint32)
    pad[:host.size] = host
    want = np.bitwise_xor.reduce(np.bitwise_xor.reduce(pad.reshape(blocks, per // 256, 256, 4), axis=3), axis=1)
    for nt in (False, True):
        sink = torch.zeros(words, dtype=torch.int32, device="cuda:0")
        dsa_gpu.ceiling_stream(src, None, sink, nontemporal=nt)
        torch.cuda.synchronize()
        assert np.array_equal(sink.cpu().numpy().view(np.uint32), want.reshape(-1))
