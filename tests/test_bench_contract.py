"""Host-side contract of bench.py: the refusal of several GPUs, and the roofline terms of the
C3 workload (2,048 newest queries over 131,072 cached keys, top_k 2,048, 64 attention heads)
against their closed forms."""
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_c3_roofline_terms():
    import bench
    import dsa_inputs as di

    wl = di.CONFIGS["C3"]
    rows = bench.workload_sizes(wl)
    assert len(rows) == 2048
    f_idx = sum(r[0] for r in rows)
    f_attn = sum(r[1] for r in rows)
    b_attn = sum(r[2] for r in rows)
    # Query t sits at position 129,024 + t and sees every key up to it; each selects 2,048 rows
    # of 576 bf16 (1,152 B), reads 4 B of index per slot, its 64 heads' 576-wide q and writes
    # their 512-wide outputs.
    n_pairs = sum(p + 1 for p in range(131072 - 2048, 131072))
    assert f_idx == 8192 * n_pairs
    assert f_attn == 2 * 64 * (576 + 512) * 2048 * 2048
    assert b_attn == 2048 * (2048 * 1152 + 4 * 2048 + 64 * 576 * 2 + 64 * 512 * 2)
    peak_flops = bench.PEAK_BF16_TFLOPS * 1e12
    peak_bytes = bench.PEAK_HBM_GBS * 1e9
    t_roof = f_idx / peak_flops + 20 * 2048 * 2048 / peak_bytes + max(f_attn / peak_flops, b_attn / peak_bytes)
    assert abs(t_roof * 1e3 - 1.525) < 1e-3  # ms; indexer 0.873 + selection 0.010 + attention 0.642


def test_topk_attention_hbm_fraction():
    """Selection + attention bytes over their kernels' time, against 8 TB/s."""
    import bench

    kernels = {"key_stats": {"ms_per_step": 0.02}, "score_sample": {"ms_per_step": 0.07},
               "row_prep": {"ms_per_step": 0.04}, "select": {"ms_per_step": 0.2},
               "fold": {"ms_per_step": 0.01}, "sparse_attention": {"ms_per_step": 0.66},
               "score_filter": {"ms_per_step": 1.6}}
    r = bench.topk_attention_hbm(kernels, 84e6, 5.13e9)
    assert r["ms_per_step"] == 1.0 and r["bytes_per_step"] == int(84e6 + 5.13e9)
    assert abs(r["achieved"] - 5214.0) < 0.1 and abs(r["frac"] - 5214.0 / 8000.0) < 1e-4
    assert "score_filter" not in r["kernels"]
    assert bench.topk_attention_hbm({"select": {"ms_per_step": 1.0}}, 1.0, 1.0) is None
