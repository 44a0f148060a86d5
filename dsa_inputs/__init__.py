"""Seeded synthetic inputs for the DSA prefill hot path.

This module only draws random numbers and rounds them to the storage types
(bf16 bit patterns as uint16, fp32, int32). It holds none of the method's
arithmetic, so both the CPU oracle's tests and the GPU path can use it.

Workloads (shapes from the five named configurations of the method's prefill
chunk, newest L positions of an N-key cache, so q_pos0 = N - L):

  name  N        L      top_k  H   indexer keys                      seed
  C0    2048     128    256    16  integers in [-4,4], w in {+-1/8,+-1/4}  0
  C1    16384    512    2048   64  N(0,1)                            1
  C2    65536    1024   2048   64  N(0,1), first 64 keys x3 (a sink) 2
  C3    131072   2048   2048   64  0.9*c + 0.1*N(0,1), c ~ N(0,I)    3
  C4    786432   8192   2048   64  as C3                             4

Indexer queries are N(0,1) and weights N(0,1)/sqrt(32) (C1..C4); attention
queries and the joined latent|rope cache are N(0,1)/24.  Draws use
numpy.random.Generator(SFC64(seed)) (PCG64 is ~10x slower on small hosts and
C4 needs ~0.9e9 normals) in the order q_idx, k_idx (c first, then the noise),
w, q, kv, as float32 in fixed chunks, then round-to-nearest-even to bf16.

A further indexer kind, "recency" (N(0,1) keys scaled by 1 + s/N), stands in for an
indexer that favours recent keys; it is a test workload, not one of the five.

"Integer twins" round the indexer draws to small integers (q in [-4,4],
k in [-12,12]) and w to {+-1/8, +-1/4} so that every fp32 score is exact.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

N_IDX_HEADS = 32
IDX_HEAD_DIM = 128
D_LATENT = 512
D_ROPE = 64
D_QK = D_LATENT + D_ROPE
SOFTMAX_SCALE = 1.0 / math.sqrt(192.0)

_CHUNK_ELEMS = 1 << 24  # float32 values drawn per call (64 MiB)


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    L: int
    top_k: int
    H: int
    seed: int
    indexer: str  # "int" | "gauss" | "sink" | "concentrated" | "recency" | "zero" | "wide"
    attention: str = "small"  # "small" = N(0,1)/24, "sharp" = q 2*N(0,1), kv N(0,1), "zero_q"
    int_twin: bool = False
    q_pos0: int | None = None  # default N - L
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def pos0(self) -> int:
        return self.N - self.L if self.q_pos0 is None else self.q_pos0

    def causal_pairs(self) -> int:
        """Number of (query, key) pairs with key <= query position."""
        p0 = self.pos0
        return sum(min(p0 + t, self.N - 1) + 1 for t in range(self.L))


CONFIGS = {
    "C0": Workload("C0", 2048, 128, 256, 16, 0, "int"),
    "C1": Workload("C1", 16384, 512, 2048, 64, 1, "gauss"),
    "C2": Workload("C2", 65536, 1024, 2048, 64, 2, "sink"),
    "C3": Workload("C3", 131072, 2048, 2048, 64, 3, "concentrated"),
    "C4": Workload("C4", 786432, 8192, 2048, 64, 4, "concentrated"),
}


def int_twin(name: str) -> Workload:
    """Same shape and seed as `name`, indexer draws rounded to small integers."""
    w = CONFIGS[name]
    return replace(w, name=name + "i", int_twin=True)


def make_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.SFC64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = u >> 16
    r &= 1
    r += 0x7FFF
    r += u  # finite inputs only: cannot wrap below 0xFF808000
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


_scratch: dict = {}


def _chunk_buffers(n: int):
    """Reusable float32/uint32 chunk buffers (fresh pages are slow on some hosts)."""
    if _scratch.get("n", 0) < n:
        _scratch["f"] = np.empty(n, np.float32)
        _scratch["u"] = np.empty(n, np.uint32)
        _scratch["n"] = n
    return _scratch["f"][:n], _scratch["u"][:n]


def _normal_f32(rng: np.random.Generator, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _CHUNK_ELEMS):
        e = min(n, s + _CHUNK_ELEMS)
        rng.standard_normal(out=out[s:e], dtype=np.float32)
    return out


def _normal_bf16(rng, shape, scale: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    sc = np.float32(scale)
    for s in range(0, n, _CHUNK_ELEMS):
        e = min(n, s + _CHUNK_ELEMS)
        x, u = _chunk_buffers(e - s)
        rng.standard_normal(out=x, dtype=np.float32)
        if scale != 1.0:
            x *= sc
        # round to nearest even into the top 16 bits (finite values only)
        xb = x.view(np.uint32)
        np.right_shift(xb, 16, out=u)
        u &= 1
        u += 0x7FFF
        u += xb
        u >>= 16
        out[s:e] = u
    return out.reshape(shape)


def make_indexer_inputs(wl: Workload, rng: np.random.Generator | None = None):
    """Returns (q_idx uint16 [L,32,128], k_idx uint16 [N,128], w float32 [L,32])."""
    if rng is None:
        rng = make_rng(wl.seed)
    L, N = wl.L, wl.N
    qshape = (L, N_IDX_HEADS, IDX_HEAD_DIM)
    kshape = (N, IDX_HEAD_DIM)
    if wl.indexer == "int":
        q = rng.integers(-4, 5, size=qshape).astype(np.float32)
        k = rng.integers(-4, 5, size=kshape).astype(np.float32)
        w = rng.choice(np.array([-0.25, -0.125, 0.125, 0.25], dtype=np.float32), size=(L, N_IDX_HEADS))
        return f32_to_bf16_bits(q), f32_to_bf16_bits(k), w.astype(np.float32)
    if wl.indexer == "zero":
        q = np.zeros(qshape, np.float32)
        k = _normal_f32(rng, N * IDX_HEAD_DIM).reshape(kshape)
        w = (_normal_f32(rng, L * N_IDX_HEADS) / np.float32(math.sqrt(32.0))).reshape(L, N_IDX_HEADS)
        return f32_to_bf16_bits(q), f32_to_bf16_bits(k), w
    q = _normal_f32(rng, L * N_IDX_HEADS * IDX_HEAD_DIM).reshape(qshape)
    if wl.indexer in ("gauss", "sink"):
        k = _normal_f32(rng, N * IDX_HEAD_DIM).reshape(kshape)
        if wl.indexer == "sink":
            k[:64] *= np.float32(3.0)
    elif wl.indexer == "wide":
        # every element scaled by its own power of two in [2^-24, 2^24]: dot products whose
        # exact value needs far more than 53 bits
        k = _normal_f32(rng, N * IDX_HEAD_DIM).reshape(kshape)
        k *= np.exp2(rng.integers(-24, 25, size=kshape)).astype(np.float32)
        q *= np.exp2(rng.integers(-24, 25, size=qshape)).astype(np.float32)
    elif wl.indexer == "recency":
        # key s scaled by 1 + s/N: key norms grow with position, so a row's largest scores
        # crowd its newest keys (about a quarter of the top 2.5 k in the newest eighth at
        # 128K keys)
        k = _normal_f32(rng, N * IDX_HEAD_DIM).reshape(kshape)
        k *= (np.float32(1.0) + np.arange(N, dtype=np.float32) / np.float32(N))[:, None]
    elif wl.indexer == "concentrated":
        c = rng.standard_normal(IDX_HEAD_DIM, dtype=np.float32)
        k = _normal_f32(rng, N * IDX_HEAD_DIM).reshape(kshape)
        k *= np.float32(0.1)
        k += np.float32(0.9) * c[None, :]
    else:
        raise ValueError(wl.indexer)
    w = _normal_f32(rng, L * N_IDX_HEADS).reshape(L, N_IDX_HEADS)
    w /= np.float32(math.sqrt(32.0))
    if wl.int_twin:
        q = np.clip(np.rint(2.0 * q), -4, 4).astype(np.float32)
        k = np.clip(np.rint(4.0 * k), -12, 12).astype(np.float32)
        med = np.median(np.abs(w))
        w = (np.sign(w) * np.where(np.abs(w) > med, 0.25, 0.125)).astype(np.float32)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), w.astype(np.float32)


def make_attention_inputs(wl: Workload, rng: np.random.Generator | None = None):
    """Returns (q uint16 [L,H,576], kv uint16 [N,576]); value = kv[:, :512]."""
    if rng is None:
        rng = make_rng(wl.seed + 1000)
    L, N, H = wl.L, wl.N, wl.H
    if wl.attention == "small":
        q = _normal_bf16(rng, (L, H, D_QK), 1.0 / 24.0)
        kv = _normal_bf16(rng, (N, D_QK), 1.0 / 24.0)
    elif wl.attention == "sharp":
        q = _normal_bf16(rng, (L, H, D_QK), 2.0)
        kv = _normal_bf16(rng, (N, D_QK), 1.0)
    elif wl.attention == "zero_q":
        q = np.zeros((L, H, D_QK), np.uint16)
        kv = _normal_bf16(rng, (N, D_QK), 1.0 / 24.0)
    else:
        raise ValueError(wl.attention)
    return q, kv


def make_inputs(wl: Workload):
    """All five inputs from one generator, drawn in the order q_idx, k_idx, w, q, kv."""
    rng = make_rng(wl.seed)
    q_idx, k_idx, w = make_indexer_inputs(wl, rng)
    q, kv = make_attention_inputs(wl, rng)
    return dict(q_idx=q_idx, k_idx=k_idx, w=w, q=q, kv=kv)


def random_topk_indices(rng: np.random.Generator, L: int, N: int, top_k: int, q_pos0: int,
                        minus_one_frac: float = 0.0, future_frac: float = 0.0) -> np.ndarray:
    """Distinct random key indices per row (for attention-only tests).

    Each row draws min(top_k, p+1) distinct causal keys in ascending order; a
    fraction of slots can be replaced by -1 or by a future key (> p) to exercise
    the skip rules.  Pure index bookkeeping, no method arithmetic.
    """
    out = np.full((L, top_k), -1, dtype=np.int32)
    for t in range(L):
        p = min(q_pos0 + t, N - 1)
        n = min(top_k, p + 1)
        sel = np.sort(rng.choice(p + 1, size=n, replace=False)).astype(np.int32)
        out[t, :n] = sel
        if minus_one_frac > 0 and n > 0:
            m = rng.random(n) < minus_one_frac
            out[t, :n][m] = -1
        if future_frac > 0 and p + 1 < N and n > 0:
            m = rng.random(n) < future_frac
            fut = rng.integers(p + 1, N, size=int(m.sum()))
            row = out[t, :n]
            row[m] = fut
    return out


def overlapping_topk_indices(rng: np.random.Generator, L: int, N: int, top_k: int, q_pos0: int,
                             keep: float) -> np.ndarray:
    """Ascending distinct causal key indices per row (-1 tail) where each row keeps about a
    fraction `keep` of the previous row's keys and draws the rest anew: neighbouring queries'
    sets overlap, as the LiteDSA packing assumes.  Pure index bookkeeping."""
    out = np.full((L, top_k), -1, dtype=np.int32)
    prev = None
    taken = np.zeros(min(q_pos0 + L, N), dtype=bool)
    for t in range(L):
        p = min(q_pos0 + t, N - 1)
        n = min(top_k, p + 1)
        kept = prev[rng.random(prev.size) < keep][:n] if prev is not None else np.zeros(0, np.int64)
        taken[kept] = True
        fresh = []
        need = n - kept.size
        while need > 0:  # draw from the causal keys not yet in the row
            cand = np.unique(rng.integers(0, p + 1, size=2 * need + 16))
            cand = cand[~taken[cand]]
            cand = cand[rng.permutation(cand.size)][:need]
            taken[cand] = True
            fresh.append(cand)
            need -= cand.size
        sel = np.sort(np.concatenate([kept] + fresh)).astype(np.int32)
        taken[sel] = False
        out[t, :n] = sel
        prev = sel
    return out
