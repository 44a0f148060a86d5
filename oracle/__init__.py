"""CPU oracle for the DSA prefill hot path -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg may
import this package.  The product library never loads it and shares no code
with it.  The arithmetic lives in ``oracle.c`` (fp64, built without FMA
contraction); ``brute.py`` holds tiny pure-Python definitions used to pin it.

Functions and the passages they follow (page titles as on the pages):
  topk(...)       -- "GLM prefill now attends only to the keys its indexer
                     picks", How it works: indexer top-k over 32 heads, full
                     argpartition or the blocked 4,096-key fold.
  scores(...)     -- the same page: the canonical score of every causal key
                     of a row (what the top-k ranks).
  causal_mask(...) -- "cuda : support for sparse KV indices in MMA flash
                     attention kernel", review: causality applied on the
                     top-k indices, masked entries -1.
  retrieval_topk(...) -- LiteTopK abstract: the same Indexer-TopK operation
                     as inner-product top-k for vector retrieval (one vector
                     per query, no ReLU, no weights, every corpus row).
  attention(...)  -- the GLM page, How it works (sparse prefill over the
                     gathered 576-wide latent|rope rows, value = latent) and
                     The change (dense boolean-masked attention).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_LIB_PATH = _HERE / "liboracle.so"
_lib = None


def build(force: bool = True) -> Path:
    """Compile oracle.c into liboracle.so (plain gcc, no fast-math, no FMA contraction)."""
    if force or not _LIB_PATH.exists():
        tmp = _LIB_PATH.with_suffix(".so.tmp")
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-pthread", "-o", str(tmp), str(_HERE / "oracle.c"), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            build(force=False)
        lib = ctypes.CDLL(str(_LIB_PATH))
        P = ctypes.c_void_p
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.dsa_oracle_score.restype = f64
        lib.dsa_oracle_score.argtypes = [P, P, P, i32, i32]
        lib.dsa_oracle_head_dots.restype = None
        lib.dsa_oracle_head_dots.argtypes = [P, P, i32, i32, P]
        lib.dsa_oracle_topk.restype = i32
        lib.dsa_oracle_topk.argtypes = [P, P, P, i64, i64, i32, i32, i64, i32, i64, P, i64, P, P, i32]
        lib.dsa_oracle_scores.restype = i32
        lib.dsa_oracle_scores.argtypes = [P, P, P, i64, i64, i32, i32, i64, P, i64, P, i32]
        lib.dsa_oracle_dot.restype = f64
        lib.dsa_oracle_dot.argtypes = [P, P, i32]
        lib.dsa_oracle_retrieval_topk.restype = i32
        lib.dsa_oracle_retrieval_topk.argtypes = [P, P, i64, i64, i32, i32, P, i64, P, P, i32]
        lib.dsa_oracle_causal_mask.restype = None
        lib.dsa_oracle_causal_mask.argtypes = [P, i64, i32, i64]
        lib.dsa_oracle_attention.restype = i32
        lib.dsa_oracle_attention.argtypes = [P, P, i64, P, i64, i64, i32, i32, i32, i32, i64, f64,
                                             i32, P, i64, P, P, i32]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    """Host threads for the oracle: the CPUs this process may run on, capped by
    OMP_NUM_THREADS when that is set (the CPU share a shared host grants one job)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def score(q_row: np.ndarray, k_row: np.ndarray, w_row: np.ndarray) -> float:
    """Canonical fp64 score of one (query, key) pair. q_row uint16 [H,d], k_row uint16 [d]."""
    q_row = np.ascontiguousarray(q_row, np.uint16)
    k_row = np.ascontiguousarray(k_row, np.uint16)
    w_row = np.ascontiguousarray(w_row, np.float32)
    H, d = q_row.shape
    return _load().dsa_oracle_score(_ptr(q_row), _ptr(k_row), _ptr(w_row), H, d)


def head_dots(q_row: np.ndarray, k_row: np.ndarray) -> np.ndarray:
    q_row = np.ascontiguousarray(q_row, np.uint16)
    k_row = np.ascontiguousarray(k_row, np.uint16)
    H, d = q_row.shape
    out = np.empty(H, np.float64)
    _load().dsa_oracle_head_dots(_ptr(q_row), _ptr(k_row), H, d, _ptr(out))
    return out


def topk(q_idx, k_idx, w, q_pos0: int, top_k: int, block: int = 0, rows=None,
         n_threads: int | None = None, return_kth: bool = False):
    """Top-k key indices per query row (ascending, -1 padded).

    q_idx uint16 [L,H,d]; k_idx uint16 [N,d]; w float32 [L,H].  block=0 is the
    full sort, block>0 the blocked fold.  rows: optional subset of rows.
    """
    q_idx = np.ascontiguousarray(q_idx, np.uint16)
    k_idx = np.ascontiguousarray(k_idx, np.uint16)
    w = np.ascontiguousarray(w, np.float32)
    L, H, d = q_idx.shape
    N = k_idx.shape[0]
    assert k_idx.shape[1] == d and w.shape == (L, H)
    if rows is not None:
        rows = np.ascontiguousarray(rows, np.int64)
        n_rows = rows.shape[0]
    else:
        n_rows = L
    out = np.empty((n_rows, top_k), np.int32)
    kth = np.empty(n_rows, np.float64) if return_kth else None
    rc = _load().dsa_oracle_topk(_ptr(q_idx), _ptr(k_idx), _ptr(w), L, N, H, d, q_pos0, top_k,
                                 block, _ptr(rows) if rows is not None else None, n_rows,
                                 _ptr(out), _ptr(kth) if kth is not None else None,
                                 n_threads or default_threads())
    if rc != 0:
        raise ValueError("oracle topk: bad arguments")
    return (out, kth) if return_kth else out


def scores(q_idx, k_idx, w, q_pos0: int, rows=None, n_threads: int | None = None) -> np.ndarray:
    """Canonical fp64 scores of the listed query rows against every key -> float64 [n_rows, N];
    NaN for keys after the row's position."""
    q_idx = np.ascontiguousarray(q_idx, np.uint16)
    k_idx = np.ascontiguousarray(k_idx, np.uint16)
    w = np.ascontiguousarray(w, np.float32)
    L, H, d = q_idx.shape
    N = k_idx.shape[0]
    assert k_idx.shape[1] == d and w.shape == (L, H)
    if rows is not None:
        rows = np.ascontiguousarray(rows, np.int64)
        n_rows = rows.shape[0]
    else:
        n_rows = L
    out = np.empty((n_rows, N), np.float64)
    rc = _load().dsa_oracle_scores(_ptr(q_idx), _ptr(k_idx), _ptr(w), L, N, H, d, q_pos0,
                                   _ptr(rows) if rows is not None else None, n_rows, _ptr(out),
                                   n_threads or default_threads())
    if rc != 0:
        raise ValueError("oracle scores: bad arguments")
    return out


def dot(a_bits: np.ndarray, b_bits: np.ndarray) -> float:
    """Canonical fp64 inner product of two bf16 rows (left to right, -0 -> +0)."""
    a = np.ascontiguousarray(a_bits, np.uint16)
    b = np.ascontiguousarray(b_bits, np.uint16)
    assert a.shape == b.shape and a.ndim == 1
    return _load().dsa_oracle_dot(_ptr(a), _ptr(b), a.shape[0])


def retrieval_topk(q, x, top_k: int, rows=None, n_threads: int | None = None, return_kth: bool = False):
    """Inner-product top-k per query row over every corpus row (ascending, -1 padded).

    q uint16 [M,d] bf16 bits; x uint16 [N,d].  Order: score desc, lower index first.
    """
    q = np.ascontiguousarray(q, np.uint16)
    x = np.ascontiguousarray(x, np.uint16)
    M, d = q.shape
    N = x.shape[0]
    assert x.shape[1] == d
    if rows is not None:
        rows = np.ascontiguousarray(rows, np.int64)
        n_rows = rows.shape[0]
    else:
        n_rows = M
    out = np.empty((n_rows, top_k), np.int32)
    kth = np.empty(n_rows, np.float64) if return_kth else None
    rc = _load().dsa_oracle_retrieval_topk(_ptr(q), _ptr(x), M, N, d, top_k,
                                           _ptr(rows) if rows is not None else None, n_rows, _ptr(out),
                                           _ptr(kth) if kth is not None else None,
                                           n_threads or default_threads())
    if rc != 0:
        raise ValueError("oracle retrieval_topk: bad arguments")
    return (out, kth) if return_kth else out


def causal_mask(idx: np.ndarray, q_pos0: int) -> np.ndarray:
    out = np.array(idx, dtype=np.int32, copy=True, order="C")
    L, k = out.shape
    _load().dsa_oracle_causal_mask(_ptr(out), L, k, q_pos0)
    return out


def attention(q, kv, idx, q_pos0: int, scale: float, d_latent: int = 512, d_rope: int = 64,
              dense: bool = False, rows=None, n_threads: int | None = None):
    """fp64 attention; returns (out [n_rows,H,d_latent], lse [n_rows,H])."""
    q = np.ascontiguousarray(q, np.uint16)
    kv = np.ascontiguousarray(kv, np.uint16)
    idx = np.ascontiguousarray(idx, np.int32)
    L, H, dqk = q.shape
    assert dqk == d_latent + d_rope
    N, stride = kv.shape
    top_k = idx.shape[1]
    assert idx.shape[0] == L
    if rows is not None:
        rows = np.ascontiguousarray(rows, np.int64)
        n_rows = rows.shape[0]
    else:
        n_rows = L
    out = np.empty((n_rows, H, d_latent), np.float64)
    lse = np.empty((n_rows, H), np.float64)
    rc = _load().dsa_oracle_attention(_ptr(q), _ptr(kv), stride, _ptr(idx), L, N, H, d_latent,
                                      d_rope, top_k, q_pos0, float(scale), 1 if dense else 0,
                                      _ptr(rows) if rows is not None else None, n_rows,
                                      _ptr(out), _ptr(lse), n_threads or default_threads())
    if rc != 0:
        raise ValueError("oracle attention: bad arguments")
    return out, lse
