"""Host-only checks of the C ABI: the library loads, exports what include/dsa.h
declares, and rejects bad arguments before touching the GPU (validation runs
before any HIP call, so these need no device)."""
import ctypes
import re
from pathlib import Path

import pytest

import dsa_sparse_attention_indexer_amd as dsa

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "dsa.h"


@pytest.fixture(scope="module")
def lib():
    if not dsa.LIB_PATH.exists():
        from dsa_sparse_attention_indexer_amd import build

        build.build()
    return dsa.load_library()


def header_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function(lib):
    names = header_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(dsa.EXPORTED)


def test_version_and_status_strings(lib):
    assert b"gfx950" in lib.dsa_version()
    assert lib.dsa_status_string(0) == b"ok"
    assert lib.dsa_status_string(3) == b"workspace too small"
    assert lib.dsa_status_string(99) == b"unknown status"


def test_gate_matches_the_glm_rule(lib):
    assert lib.dsa_sparse_prefill_gate(1, 512, 16384, 0) == 1
    assert lib.dsa_sparse_prefill_gate(1, 512, 16383, 0) == 0  # below the minimum context
    assert lib.dsa_sparse_prefill_gate(2, 512, 131072, 0) == 0  # batches stay dense
    assert lib.dsa_sparse_prefill_gate(1, 1, 131072, 0) == 0  # decode untouched
    assert lib.dsa_sparse_prefill_gate(1, 2, 4096, 4096) == 1


def test_workspace_is_bounded_by_the_query_block(lib):
    ws = lib.dsa_indexer_topk_workspace_bytes
    a = ws(2048, 131072, 2048, 1024)
    b = ws(8192, 131072, 2048, 1024)
    assert a == b > 0  # independent of L beyond one block
    assert ws(1024, 131072, 2048, 1024) == a
    assert ws(512, 131072, 2048, 1024) < a
    assert ws(1024, 131072, 2048, 256) < a
    # grows with N only through the threshold sample, never as L*N
    big = ws(8192, 786432, 2048, 1024)
    assert big < 8192 * 786432 * 4 / 50
    assert ws(-1, 100, 1, 0) == 0 and ws(1, 0, 1, 0) == 0 and ws(1, 100, 0, 0) == 0
    assert ws(1, 100, dsa.MAX_TOPK + 1, 0) == 0


NULL = None


def call_indexer(lib, L=4, N=64, nh=32, hd=128, q_pos0=60, k=8, qb=0, ptr=1 << 20, ws=1 << 30,
                 ws_bytes=1 << 40):
    p = ctypes.c_void_p(ptr) if ptr else None
    return lib.dsa_indexer_topk(p, p, p, L, N, nh, hd, q_pos0, k, qb, p,
                                ctypes.c_void_p(ws) if ws else None, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(L=-1), 1), (dict(N=0), 1), (dict(q_pos0=-1), 1), (dict(q_pos0=61), 1),
    (dict(k=0), 1), (dict(k=4097), 1), (dict(qb=-2), 1),
    (dict(nh=16), 2), (dict(hd=64), 2), (dict(ptr=0), 1),
    (dict(ws=0), 3), (dict(ws_bytes=10), 3), (dict(ptr=(1 << 20) + 2), 1),
])
def test_indexer_rejects_bad_arguments(lib, kw, status):
    assert call_indexer(lib, **kw) == status
    assert lib.dsa_last_error() != b""


def test_indexer_zero_rows_is_a_no_op(lib):
    assert call_indexer(lib, L=0, ptr=0, ws=0, ws_bytes=0) == 0


def call_attn(lib, L=4, N=64, H=64, dl=512, dr=64, k=8, q_pos0=60, stride=576, scale=0.07, qb=0,
              ptr=1 << 20):
    p = ctypes.c_void_p(ptr) if ptr else None
    return lib.dsa_sparse_prefill(p, p, stride, p, L, N, H, dl, dr, k, q_pos0, scale, qb, p, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(L=-1), 1), (dict(N=0), 1), (dict(q_pos0=61), 1), (dict(k=0), 1), (dict(qb=-1), 1),
    (dict(H=24), 2), (dict(H=0), 2), (dict(H=144), 2), (dict(dl=256), 2), (dict(dr=32), 2),
    (dict(stride=575), 1), (dict(stride=580), 1), (dict(scale=float("nan")), 1),
    (dict(scale=float("inf")), 1), (dict(ptr=0), 1),
])
def test_attention_rejects_bad_arguments(lib, kw, status):
    assert call_attn(lib, **kw) == status
    assert lib.dsa_last_error() != b""


def test_attention_zero_rows_is_a_no_op(lib):
    assert call_attn(lib, L=0, ptr=0) == 0


def call_decode(lib, L=1, N=64, H=64, dl=512, dr=64, k=64, q_pos0=63, stride=576, scale=0.07, splits=0,
                ptr=1 << 20, ws=1 << 24, ws_bytes=1 << 30):
    p = ctypes.c_void_p(ptr) if ptr else None
    w = ctypes.c_void_p(ws) if ws else None
    return lib.dsa_sparse_decode(p, p, stride, p, L, N, H, dl, dr, k, q_pos0, scale, splits, p, None,
                                 w, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(L=-1), 1), (dict(N=0), 1), (dict(q_pos0=64), 1), (dict(k=0), 1), (dict(splits=-1), 1),
    (dict(splits=129), 1), (dict(H=24), 2), (dict(H=144), 2), (dict(dl=256), 2), (dict(dr=32), 2),
    (dict(stride=575), 1), (dict(scale=float("nan")), 1), (dict(ptr=0), 1),
    (dict(ws=0), 3), (dict(ws_bytes=1024), 3), (dict(ws=(1 << 24) + 16), 1),
])
def test_decode_rejects_bad_arguments(lib, kw, status):
    assert call_decode(lib, **kw) == status
    assert lib.dsa_last_error() != b""


def test_decode_zero_rows_is_a_no_op(lib):
    assert call_decode(lib, L=0, ptr=0, ws=0, ws_bytes=0) == 0


def test_decode_workspace_size():
    import dsa_sparse_attention_indexer_amd as d

    lib = d.load_library()
    f = lib.dsa_sparse_decode_workspace_bytes
    # explicit splits: rows x splits x H x (512 + 4) fp32
    assert f(1, 64, 2048, 8) == 1 * 8 * 64 * 516 * 4
    # splits are clamped to the tile count of top_k (32 keys per tile)
    assert f(1, 64, 64, 8) == 1 * 2 * 64 * 516 * 4
    # automatic: about 512 workgroups, at most one tile each and at most 128 splits
    assert f(1, 64, 2048, 0) == 1 * 64 * 64 * 516 * 4
    assert f(4, 16, 8192, 0) == 4 * 128 * 16 * 516 * 4
    assert f(1024, 64, 2048, 0) == 1024 * 1 * 64 * 516 * 4
    # partials of at most 1,024 queries
    assert f(5000, 64, 2048, 2) == 1024 * 2 * 64 * 516 * 4
    assert f(0, 64, 2048, 0) == 0
    assert f(1, 24, 2048, 0) == 0 and f(1, 64, 0, 0) == 0 and f(1, 64, 2048, 129) == 0


def test_causal_mask_rejects_bad_arguments(lib):
    f = lib.dsa_causal_mask_topk
    assert f(ctypes.c_void_p(1 << 20), -1, 4, 0, None) == 1
    assert f(ctypes.c_void_p(1 << 20), 4, 0, 0, None) == 1
    assert f(ctypes.c_void_p(1 << 20), 4, 4, -1, None) == 1
    assert f(None, 4, 4, 0, None) == 1
    assert f(None, 0, 4, 0, None) == 0


def test_python_binding_raises_without_library(monkeypatch, tmp_path):
    import importlib

    mod = importlib.reload(dsa)
    try:
        monkeypatch.setattr(mod, "LIB_PATH", tmp_path / "missing.so")
        with pytest.raises(RuntimeError, match="missing"):
            mod.load_library()
    finally:
        importlib.reload(dsa)


# ------------------------------------------------------------------ batched (varlen) entry points

def i64s(vals):
    return (ctypes.c_int64 * max(len(vals), 1))(*vals)


GOOD_BATCH = dict(cu_q=[0, 70, 71, 584], cu_k=[0, 5000, 25000, 28000], pos0=[100, 30, 2487])


def call_indexer_varlen(lib, cu_q=None, cu_k=None, pos0=None, B=None, nh=32, hd=128, k=64, qb=0, ptr=1 << 20,
                        ws=1 << 30, ws_bytes=1 << 40, arrays=True):
    cu_q = GOOD_BATCH["cu_q"] if cu_q is None else cu_q
    cu_k = GOOD_BATCH["cu_k"] if cu_k is None else cu_k
    pos0 = GOOD_BATCH["pos0"] if pos0 is None else pos0
    B = len(pos0) if B is None else B
    p = ctypes.c_void_p(ptr) if ptr else None
    a = (i64s(cu_q), i64s(cu_k), i64s(pos0)) if arrays else (None, None, None)
    return lib.dsa_indexer_topk_varlen(p, p, p, B, *a, nh, hd, k, qb, p, ctypes.c_void_p(ws) if ws else None,
                                       ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), 1), (dict(B=dsa.MAX_BATCH + 1), 1), (dict(arrays=False), 1),
    (dict(cu_q=[1, 70, 71, 584]), 1), (dict(cu_k=[5, 5000, 25000, 28000]), 1),
    (dict(cu_q=[0, 70, 69, 584]), 1), (dict(cu_k=[0, 5000, 4000, 28000]), 1),
    (dict(pos0=[100, -1, 2487]), 1), (dict(pos0=[100, 30, 2488]), 1),  # pos0 + L > N
    (dict(k=0), 1), (dict(k=4097), 1), (dict(qb=-1), 1), (dict(nh=16), 2), (dict(hd=64), 2),
    (dict(ptr=0), 1), (dict(ptr=(1 << 20) + 2), 1), (dict(ws=0), 3), (dict(ws_bytes=1000), 3),
])
def test_indexer_varlen_rejects_bad_arguments(lib, kw, status):
    assert call_indexer_varlen(lib, **kw) == status
    assert lib.dsa_last_error() != b""


def test_indexer_varlen_without_query_rows_is_a_no_op(lib):
    assert call_indexer_varlen(lib, cu_q=[0], cu_k=[0], pos0=[], ptr=0, ws=0, ws_bytes=0) == 0
    assert call_indexer_varlen(lib, cu_q=[0, 0, 0], cu_k=[0, 0, 9], pos0=[0, 9], ptr=0, ws=0, ws_bytes=0) == 0


def test_indexer_varlen_workspace(lib):
    f = lib.dsa_indexer_topk_varlen_workspace_bytes
    ws = lambda cq, ck, p0, k=2048, qb=1024: f(len(p0), i64s(cq), i64s(ck), i64s(p0), k, qb)
    one = ws([0, 2048], [0, 131072], [129024])
    # one sequence: the single-sequence figure plus its row table (2048 x 40 B) and key table entry
    assert one >= lib.dsa_indexer_topk_workspace_bytes(2048, 131072, 2048, 1024)
    assert one - lib.dsa_indexer_topk_workspace_bytes(2048, 131072, 2048, 1024) <= 2048 * 40 + 512
    # rejected batches and batches without rows size to 0
    assert ws([0, 5], [0, 4], [0]) == 0 and ws([0], [0], []) == 0 and ws([0, 0], [0, 9], [3]) == 0
    assert ws([0, 70], [0, 5000], [0], k=0) == 0
    # the tiled key copies cover only the keys queries can see
    a = ws([0, 8], [0, 100000], [0])
    b = ws([0, 8], [0, 100000], [99992])
    assert b - a >= (100000 // 32 - 1) * 8192


def call_attn_varlen(lib, cu_q=None, cu_k=None, pos0=None, H=64, dl=512, dr=64, k=8, stride=576, scale=0.07,
                     splits=1, ptr=1 << 20, ws=1 << 24, ws_bytes=1 << 30):
    cu_q = GOOD_BATCH["cu_q"] if cu_q is None else cu_q
    cu_k = GOOD_BATCH["cu_k"] if cu_k is None else cu_k
    pos0 = GOOD_BATCH["pos0"] if pos0 is None else pos0
    p = ctypes.c_void_p(ptr) if ptr else None
    return lib.dsa_sparse_prefill_varlen(p, p, stride, p, len(pos0), i64s(cu_q), i64s(cu_k), i64s(pos0), H, dl, dr,
                                         k, scale, splits, p, None, ctypes.c_void_p(ws) if ws else None, ws_bytes,
                                         None)


@pytest.mark.parametrize("kw,status", [
    (dict(cu_q=[0, 70, 69, 584]), 1), (dict(pos0=[100, 30, 2488]), 1), (dict(k=0), 1), (dict(splits=-1), 1),
    (dict(splits=129), 1), (dict(H=24), 2), (dict(dl=256), 2), (dict(dr=32), 2), (dict(stride=575), 1),
    (dict(scale=float("nan")), 1), (dict(ptr=0), 1), (dict(ws=0), 3), (dict(ws_bytes=64), 3),
    (dict(ws=(1 << 24) + 16), 1),
])
def test_attention_varlen_rejects_bad_arguments(lib, kw, status):
    assert call_attn_varlen(lib, **kw) == status
    assert lib.dsa_last_error() != b""


def test_attention_varlen_workspace(lib):
    f = lib.dsa_sparse_prefill_varlen_workspace_bytes
    c = GOOD_BATCH
    args = (3, i64s(c["cu_q"]), i64s(c["cu_k"]), i64s(c["pos0"]))
    T = c["cu_q"][-1]
    table = (T * 16 + 255) // 256 * 256
    assert f(*args, 64, 2048, 1) == table  # the per-query table only
    assert f(*args, 64, 2048, 4) == table + T * 4 * 64 * 516 * 4
    assert f(*args, 24, 2048, 1) == 0 and f(*args, 64, 2048, 129) == 0
    assert call_attn_varlen(lib, cu_q=[0], cu_k=[0], pos0=[], ptr=0, ws=0, ws_bytes=0) == 0


# ------------------------------------------------------------------ vector retrieval

def call_retrieval(lib, M=4, N=64, dim=128, k=8, qb=0, ptr=1 << 20, ws=1 << 30, ws_bytes=1 << 40):
    p = ctypes.c_void_p(ptr) if ptr else None
    return lib.dsa_retrieval_topk(p, p, M, N, dim, k, qb, p, ctypes.c_void_p(ws) if ws else None, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), 1), (dict(N=0), 1), (dict(N=1 << 31), 2), (dict(k=0), 1), (dict(k=4097), 1), (dict(qb=-1), 1),
    (dict(dim=64), 2), (dict(ptr=0), 1), (dict(ptr=(1 << 20) + 8), 1), (dict(ws=0), 3), (dict(ws_bytes=100), 3),
    (dict(ws=(1 << 30) + 16), 1),
])
def test_retrieval_rejects_bad_arguments(lib, kw, status):
    assert call_retrieval(lib, **kw) == status
    assert lib.dsa_last_error() != b""


def test_retrieval_zero_queries_and_workspace(lib):
    assert call_retrieval(lib, M=0, ptr=0, ws=0, ws_bytes=0) == 0
    f = lib.dsa_retrieval_topk_workspace_bytes
    a, b = f(1024, 1 << 20, 1024, 0), f(4096, 1 << 20, 1024, 0)
    assert a == b > 0  # bounded by the query block
    # no copy of the corpus: beyond a million rows the size hardly depends on N
    assert f(1024, 4 << 20, 1024, 0) < 1.2 * f(1024, 1 << 20, 1024, 0)
    assert f(0, 100, 8, 0) == 0 and f(4, 0, 8, 0) == 0 and f(4, 100, 0, 0) == 0 and f(4, 100, 8, -1) == 0


def test_profile_set_validates_names(lib):
    assert lib.dsa_profile_set(b"score_filter,sparse_attention") == 0
    assert lib.dsa_profile_set(b"score_filter,bogus") == 1
    assert b"bogus" in lib.dsa_last_error()
    assert lib.dsa_profile_set(b"") == 0 and lib.dsa_profile_set(None) == 0
    assert lib.dsa_profile_enable(0) == 0


def test_stats_rejects_bad_arguments(lib):
    st = dsa.IndexerStats()
    f = lib.dsa_indexer_topk_stats
    assert f(None, ctypes.byref(st), None) == 1
    assert f(ctypes.c_void_p((1 << 20) + 16), ctypes.byref(st), None) == 1  # not 256-byte aligned
    assert f(ctypes.c_void_p(1 << 20), None, None) == 1


def call_scores(lib, L=4, N=64, nh=32, hd=128, q_pos0=60, ptr=1 << 20, ws=1 << 30, ws_bytes=1 << 40):
    p = ctypes.c_void_p(ptr) if ptr else None
    return lib.dsa_indexer_scores(p, p, p, L, N, nh, hd, q_pos0, p, p,
                                  ctypes.c_void_p(ws) if ws else None, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(L=65, N=200, q_pos0=100), 1), (dict(q_pos0=0), 1), (dict(q_pos0=61), 1), (dict(nh=16), 2),
    (dict(ptr=0), 1), (dict(ws=0), 3), (dict(ws_bytes=10), 3), (dict(ws=(1 << 30) + 8), 1),
])
def test_scores_rejects_bad_arguments(lib, kw, status):
    assert call_scores(lib, **kw) == status
    assert lib.dsa_last_error() != b""


def test_scores_workspace(lib):
    f = lib.dsa_indexer_scores_workspace_bytes
    assert f(0, 100) == 0 and f(dsa.MAX_SCORE_ROWS + 1, 100) == 0 and f(4, 0) == 0
    # every key of every (row-group-padded) row fits as a candidate
    assert f(8, 131072) > 8 * 131072 * 8
    assert f(1, 1000) == f(8, 1000)


def test_noalloc_rejects_before_touching_the_device(lib):
    p = ctypes.c_void_p(1 << 20)
    f = lib.dsa_indexer_topk_noalloc
    # a C3 chunk in one 2,048-query block needs more than the static scratch
    assert lib.dsa_indexer_topk_workspace_bytes(2048, 131072, 2048, 2048) > dsa.NOALLOC_SCRATCH_BYTES
    assert f(p, p, p, 2048, 131072, 32, 128, 129024, 2048, 2048, p, None) == 3
    assert b"static scratch" in lib.dsa_last_error()
    assert f(p, p, p, 4, 64, 16, 128, 60, 8, 0, p, None) == 2   # the indexer's own checks first
    assert f(None, None, None, 0, 64, 32, 128, 0, 8, 0, None, None) == 0  # L = 0: no-op


def test_key_cache_rejects_bad_arguments(lib):
    p = ctypes.c_void_p(1 << 20)
    assert lib.dsa_indexer_key_cache_bytes(0) == 0
    n = lib.dsa_indexer_key_cache_bytes(100)
    assert n >= 256 + 4 * 32 * 128 * 2  # header and four 32-key tiles
    f = lib.dsa_indexer_key_cache_append
    assert f(p, 5, 4, p, n, None) == 1            # n_new < n_old
    assert f(p, 0, 10, None, n, None) == 1        # no cache
    assert f(p, 0, 10, ctypes.c_void_p((1 << 20) + 64), n, None) == 1  # unaligned cache
    assert f(p, 0, 200, p, n, None) == 1          # too small for 200 keys
    assert f(None, 0, 10, p, n, None) == 1        # no keys to append
    g = lib.dsa_indexer_topk_cached
    ws = lib.dsa_indexer_topk_cached_workspace_bytes(4, 64, 8, 0)
    assert 0 < ws < lib.dsa_indexer_topk_workspace_bytes(4, 64, 8, 0)  # no key copy in it
    args = (p, p, p, 4, 64, 32, 128, 60, 8, 0, p)
    assert g(*args, None, n, 64, p, ws, None) == 1          # no cache
    assert g(*args, p, n, 63, p, ws, None) == 1             # cache holds fewer keys than the queries see
    assert g(*args, p, n, 65, p, ws, None) == 1             # more keys than N
    assert g(*args, p, 16, 64, p, ws, None) == 1            # cache buffer too small
    assert g(*args, p, n, 64, p, 10, None) == 3             # workspace too small


def test_ceilings_reject_bad_arguments(lib):
    """The measured-ceiling kernels validate before touching the GPU."""
    fl = ctypes.c_double()
    p = ctypes.c_void_p(1 << 20)
    f = lib.dsa_ceiling_mfma_bf16
    assert f(p, 1 << 20, 10, 1, 3, ctypes.byref(fl), None) == 1  # waves per SIMD 1 or 2
    assert f(p, 1 << 20, 0, 1, 1, ctypes.byref(fl), None) == 1  # iters >= 1
    assert f(None, 1 << 20, 10, 1, 1, ctypes.byref(fl), None) == 1
    assert f(p, 1 << 20, 10, 1, 1, None, None) == 1
    assert lib.dsa_ceiling_mfma_threads(3) == 0
    c = lib.dsa_ceiling_stream
    assert c(None, p, 1024, None, 0, 0, None) == 1
    assert c(p, ctypes.c_void_p((1 << 20) + 8), 1024, None, 0, 0, None) == 1  # 16-byte alignment
    assert c(p, p, 1000, None, 0, 0, None) == 1  # a multiple of 16 bytes
    assert c(p, None, 1024, None, 0, 0, None) == 1  # a read-only stream needs a sink
    assert c(p, None, 1024, p, lib.dsa_ceiling_stream_sink_words() - 1, 0, None) == 1
    assert c(p, p, 0, None, 0, 0, None) == 0  # nothing to stream
    assert "ceiling_mfma" in dsa.PROFILE_KERNELS and "ceiling_copy" in dsa.PROFILE_KERNELS
    assert lib.dsa_profile_set(b"ceiling_mfma,ceiling_copy") == 0
    assert lib.dsa_profile_enable(0) == 0
