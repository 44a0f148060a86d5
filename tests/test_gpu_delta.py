"""The error bound behind the exact selection, measured on the production scoring kernel.

The selection ranks keys by the canonical fp64 score; the GPU's fp32 matrix-core scores
only pick candidates, and every key whose fp32 score lies within 2 delta_t of the k-th is
re-scored in fp64 (the GLM page, How it works: the sparse path selects the same keys as the
stock indexer; the LiteTopK abstract: exact top-k).  That is exact only if

    |s32(t, s) - s64(t, s)| <= delta_t = 104 * u_t  for every key s,
    u_t = 2^-24 * max_s ||k_s||_2 * sum_h |w_th| ||q_th||_2.

dsa_indexer_scores returns the fp32 scores of the scoring kernel (the filter, with its
threshold at -inf so it keeps every causal key) and the delta_t it uses.  Each case
compares them with the oracle's fp64 scores on every causal key of 8 rows, asserts the
largest error stays under delta_t / 2 (a factor-2 margin), and prints the observed
coefficient max|s32 - s64| / u_t.  Rows that are provably exact (integer inputs) must have
delta_t = 0 and s32 == s64 bit for bit.
"""
import numpy as np
import pytest

import dsa_inputs as di
from tests.gpu_util import report, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

DELTA_COEF = 104.0


def unit(q, k, w, n_keys):
    """u_t = 2^-24 max_s ||k_s|| sum_h |w_h| ||q_h|| for each row (fp64)."""
    kf = di.bf16_bits_to_f32(k[:n_keys]).astype(np.float64)
    knorm = np.sqrt((kf * kf).sum(axis=1)).max()
    qf = di.bf16_bits_to_f32(q).astype(np.float64)
    qn = np.sqrt((qf * qf).sum(axis=2))  # [rows, heads]
    return 2.0 ** -24 * knorm * (np.abs(w.astype(np.float64)) * qn).sum(axis=1)


def measure(dsa, oracle_mod, q, k, w, q_pos0, what, exact=False):
    import torch

    L = q.shape[0]
    s32_d, delta_d = dsa.indexer_scores(to_dev_bf16(q), to_dev_bf16(k), to_dev(w), q_pos0)
    torch.cuda.synchronize()
    s32 = s32_d.cpu().numpy().astype(np.float64)
    delta = delta_d.cpu().numpy().astype(np.float64)
    s64 = oracle_mod.scores(q, k, w, q_pos0)
    causal = np.arange(k.shape[0])[None, :] <= (q_pos0 + np.arange(L))[:, None]
    assert np.array_equal(np.isnan(s32), ~causal), f"{what}: scores missing or past the position"
    err = np.where(causal, np.abs(s32 - s64), 0.0).max(axis=1)
    if exact:
        assert (delta == 0).all(), f"{what}: exact rows must have delta = 0"
        assert (err == 0).all(), f"{what}: exact rows differ from the fp64 scores"
        report(f"{what}: {L} rows exact (delta 0, fp32 == fp64 on every key)")
        return 0.0
    u = unit(q, k, w, q_pos0 + L)
    coef = err / u
    # the kernel's delta is the formula's, up to the rounding-up of its inputs
    assert (delta >= DELTA_COEF * u * (1 - 1e-6)).all() and (delta <= DELTA_COEF * u * 1.001).all(), what
    report(f"{what}: max|s32-s64|/u per row = {np.round(coef, 3).tolist()} "
           f"(max {coef.max():.3f}; delta = {DELTA_COEF:g} u)")
    assert (err <= delta / 2).all(), f"{what}: error {err.max():.3g} above delta/2 ({coef.max():.2f} u)"
    return float(coef.max())


def rows_of(wl, r0, n=8):
    q, k, w = di.make_indexer_inputs(wl)
    return q[r0:r0 + n], k, w[r0:r0 + n], wl.pos0 + r0


@pytest.mark.parametrize("name,r0", [("C1", 0), ("C1", 504), ("C2", 0), ("C2", 1016), ("C3", 0),
                                     ("C3", 2040)])
def test_config_rows(dsa_gpu, oracle_mod, name, r0):
    q, k, w, p0 = rows_of(di.CONFIGS[name], r0)
    measure(dsa_gpu, oracle_mod, q, k, w, p0, f"{name} rows {r0}..{r0 + 7}")


def test_c4_rows(dsa_gpu, oracle_mod):
    wl = di.CONFIGS["C4"]
    q, k, w = di.make_indexer_inputs(wl)
    r0 = 8184
    measure(dsa_gpu, oracle_mod, q[r0:], k, w[r0:], wl.pos0 + r0, "C4 rows 8184..8191")


@pytest.mark.parametrize("name", ["C0", "C1i", "C3i"])
def test_exact_rows(dsa_gpu, oracle_mod, name):
    wl = di.CONFIGS["C0"] if name == "C0" else di.int_twin(name[:2])
    q, k, w, p0 = rows_of(wl, wl.L - 8)
    measure(dsa_gpu, oracle_mod, q, k, w, p0, name, exact=True)


def test_wide_dynamic_range(dsa_gpu, oracle_mod):
    """Every element scaled by its own 2^-24 .. 2^24."""
    wl = di.Workload("wide", 4096, 8, 64, 16, 31, "wide")
    q, k, w = di.make_indexer_inputs(wl)
    measure(dsa_gpu, oracle_mod, q, k, w, wl.pos0, "wide dynamic range")


def test_large_magnitude(dsa_gpu, oracle_mod):
    """Gaussian inputs scaled by 2^40 (q) and 2^36 (k): scores near 2^80, far from fp32's limits."""
    wl = di.Workload("big", 4096, 8, 64, 16, 32, "gauss")
    q, k, w = di.make_indexer_inputs(wl)
    q = di.f32_to_bf16_bits(di.bf16_bits_to_f32(q) * np.float32(2.0 ** 40))
    k = di.f32_to_bf16_bits(di.bf16_bits_to_f32(k) * np.float32(2.0 ** 36))
    measure(dsa_gpu, oracle_mod, q, k, w, wl.pos0, "large magnitude")


@pytest.mark.parametrize("pattern", ["aligned", "alternating"])
def test_adversarial_accumulation(dsa_gpu, oracle_mod, pattern):
    """Head h of every row is a copy of key s_h (elements of spread exponents): its dot
    product with that key sums 128 positive products whose partial sums keep growing
    ("aligned"), or the same products with alternating signs, so the partial sums swing and
    cancel ("alternating").  Positive weights keep those heads in the score."""
    rng = np.random.default_rng(41)
    N, L = 4096, 8
    kf = rng.standard_normal((N, 128)).astype(np.float32) * np.exp2(rng.integers(-6, 7, size=(N, 128))).astype(np.float32)
    k = di.f32_to_bf16_bits(kf)
    src = rng.choice(N - L, size=(L, 32), replace=False)
    qf = di.bf16_bits_to_f32(k)[src]  # [L, 32, 128]
    if pattern == "alternating":
        qf = qf * np.where(np.arange(128) % 2 == 0, 1.0, -1.0).astype(np.float32)
    q = di.f32_to_bf16_bits(qf)
    w = np.abs(rng.standard_normal((L, 32))).astype(np.float32) / np.float32(np.sqrt(32.0))
    measure(dsa_gpu, oracle_mod, q, k, w, N - L, f"adversarial {pattern}")
