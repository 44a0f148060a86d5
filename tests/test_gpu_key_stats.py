"""The indexer's key statistics and tiled key copy, read back from an append-only key cache.

The error bound behind the exact selection (delta = 104 * 2^-24 * max ||k_s|| * ..) and
the exactness tests of the fp64 re-score (the product range against the lowest set bit)
rest on three statistics of the keys, which the key-statistics kernel computes while it
lays the keys out in the scoring kernel's tile order.  A key cache (dsa_indexer_key_cache_*)
keeps them in its 256-byte header: the largest key norm (fp32, rounded up), the largest
element magnitude (fp32) and the lowest exponent of any nonzero element's lowest set bit.
Here they are checked against their definitions (numpy, fp64), and the tiled copy against
the tile order written out directly:
- norm: at least the largest fp64 norm, and at most 2^-13 above it;
- magnitude and lowest-set-bit exponent: exact;
- tile t, 16-byte chunk i * 64 + l: key 32 t + (l % 32), dims 64 (l // 32) + 8 i ..,
  zero past the last key.
Inputs: Gaussian keys, integer keys with zeros, keys spread over 2^-60 .. 2^60 with bf16
subnormals planted, all-zero keys, and a cache grown by chunks that end inside a tile
(the partial tile is laid out again, and the statistics merge).
"""
import numpy as np
import pytest

import dsa_inputs as di
from tests.gpu_util import report, to_dev_bf16

pytestmark = pytest.mark.gpu

HEADER = 256
TILE_KEYS = 32


def lowest_bit_exponent(bits: np.ndarray) -> int:
    """min over nonzero bf16 elements of the exponent of their lowest set bit, or None."""
    mag = (bits & 0x7FFF).astype(np.int64)
    mag = mag[mag != 0]
    if mag.size == 0:
        return None
    e = mag >> 7
    m = mag & 0x7F
    sig = np.where(e > 0, m | 0x80, m)  # integer significand: value = sig * 2^(max(e,1) - 134)
    tz = np.zeros_like(sig)
    s = sig.copy()
    while (s & 1 == 0).any():
        even = (s & 1) == 0
        tz += even
        s = np.where(even, s >> 1, s)
    return int((np.maximum(e, 1) - 134 + tz).min())


def expected_tiles(bits: np.ndarray) -> np.ndarray:
    n = bits.shape[0]
    n_tiles = (n + TILE_KEYS - 1) // TILE_KEYS
    pad = np.zeros((n_tiles * TILE_KEYS, 128), np.uint16)
    pad[:n] = bits
    keys = pad.reshape(n_tiles, TILE_KEYS, 2, 8, 8)  # [tile, key c, half, chunk i, 8 dims]
    # chunk index i * 64 + 32 * half + c
    return keys.transpose(0, 3, 2, 1, 4).reshape(n_tiles, -1)


def read_cache(cache, n):
    import torch

    torch.cuda.synchronize()
    raw = cache.buffer.cpu().numpy()
    head = raw[:16].view(np.uint32)
    n_tiles = (n + TILE_KEYS - 1) // TILE_KEYS
    tiles = raw[HEADER:HEADER + n_tiles * TILE_KEYS * 256].view(np.uint16).reshape(n_tiles, -1)
    knorm = float(head[0:1].view(np.float32)[0])
    kinf = float(head[1:2].view(np.float32)[0])
    kexp = int(head[2:3].view(np.int32)[0])
    return knorm, kinf, kexp, tiles


def check(cache, bits, what):
    n = bits.shape[0]
    knorm, kinf, kexp, tiles = read_cache(cache, n)
    f = di.bf16_bits_to_f32(bits).astype(np.float64)
    true_norm = np.sqrt((f * f).sum(axis=1)).max()
    assert knorm >= true_norm, f"{what}: norm {knorm} below {true_norm}"
    assert knorm <= true_norm * (1 + 2.0 ** -13) + 1e-300, f"{what}: norm {knorm} too loose ({true_norm})"
    assert kinf == np.abs(f).max(), f"{what}: max magnitude {kinf} vs {np.abs(f).max()}"
    want_e = lowest_bit_exponent(bits)
    assert kexp == (2 ** 31 - 1 if want_e is None else want_e), f"{what}: lowest bit exponent {kexp} vs {want_e}"
    assert np.array_equal(tiles, expected_tiles(bits)), f"{what}: tiled copy differs"
    report(f"{what}: {n} keys, norm {knorm:.6g} (true {true_norm:.6g}), max {kinf:.6g}, lowest bit 2^{kexp}")


def cases():
    rng = np.random.default_rng(77)
    gauss = di.f32_to_bf16_bits(rng.standard_normal((5000, 128), dtype=np.float32))
    ints = di.f32_to_bf16_bits(rng.integers(-3, 4, size=(777, 128)).astype(np.float32))
    # element scales 2^-60 .. 2^60 (the squares stay within fp32's normal range), plus
    # elements far below it, which do not move the norm but set the lowest bit
    wide = rng.standard_normal((1000, 128)).astype(np.float32)
    wide = wide * np.exp2(rng.integers(-60, 61, size=(1000, 128))).astype(np.float32)
    wide = di.f32_to_bf16_bits(wide)
    wide[3, 5] = 0x0001  # the smallest bf16 subnormal, 2^-133
    wide[5, 6] = 0x8043  # -(0x43) * 2^-133, a subnormal with its lowest set bit at 2^-133
    wide[6, 7] = 0x0380  # 2^-120, a power of two (lowest set bit: the implicit one)
    wide[7, 9] = 0x8000  # -0
    zeros = np.zeros((40, 128), np.uint16)
    one = di.f32_to_bf16_bits(np.full((1, 128), 0.75, np.float32))
    return {"gauss": gauss, "integers": ints, "wide": wide, "zeros": zeros, "one key": one}


@pytest.mark.parametrize("name", ["gauss", "integers", "wide", "zeros", "one key"])
def test_statistics_and_tiles(dsa_gpu, name):
    bits = cases()[name]
    cache = dsa_gpu.KeyCache(bits.shape[0])
    cache.append(to_dev_bf16(bits))
    check(cache, bits, name)


def test_chunked_growth_merges(dsa_gpu):
    """Chunks ending inside tiles; the largest norm, the largest element and the lowest bit
    each sit in a different chunk."""
    rng = np.random.default_rng(78)
    f = rng.standard_normal((3000, 128)).astype(np.float32)
    f[1500] *= 8.0      # largest norm
    f[100, 3] = 40.0    # largest element
    f[2900, 7] = 2.0 ** -90 * 1.5  # lowest set bit 2^-91
    bits = di.f32_to_bf16_bits(f)
    kd = to_dev_bf16(bits)
    cache = dsa_gpu.KeyCache(bits.shape[0])
    for n in (101, 133, 1501, 1502, 2000, 2901, 3000):
        cache.append(kd, n)
        check(cache, bits[:n], f"chunked to {n}")
