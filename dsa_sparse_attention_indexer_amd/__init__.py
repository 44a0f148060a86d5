"""DeepSeek-sparse-attention prefill hot path on MI355X (gfx950).

Thin Python binding over libdsa.so (include/dsa.h).  This module only marshals
arguments: every step of the path runs in the HIP kernels of the library, and
PyTorch supplies device memory and the current stream.  There is no CPU or
PyTorch fallback; calling any op without the built library raises.

    idx = indexer_topk(q_idx, k_idx, w, q_pos0, top_k)       # int32 [L, top_k]
    out = sparse_prefill(q, kv, idx, q_pos0, scale)          # bf16  [L, H, 512]

A batch of sequences of any lengths goes through the *_varlen calls, described by
host-side cu_q / cu_k offsets and per-sequence start positions pos0.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libdsa.so"

DSA_OK = 0
STATUS_NAMES = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED",
                3: "DSA_ERR_WORKSPACE", 4: "DSA_ERR_HIP"}
INDEX_HEADS = 32
INDEX_DIM = 128
MAX_TOPK = 4096
D_LATENT = 512
D_ROPE = 64
DEFAULT_Q_BLOCK = 1024
MAX_BATCH = 65536
MAX_SCORE_ROWS = 64
NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTED = ["dsa_indexer_topk_workspace_bytes", "dsa_indexer_topk", "dsa_causal_mask_topk",
            "dsa_sparse_prefill", "dsa_sparse_prefill_packed", "dsa_sparse_decode_workspace_bytes",
            "dsa_sparse_decode",
            "dsa_indexer_topk_noalloc", "dsa_indexer_key_cache_bytes", "dsa_indexer_key_cache_append",
            "dsa_indexer_topk_cached_workspace_bytes", "dsa_indexer_topk_cached", "dsa_indexer_topk_stats", "dsa_indexer_scores_workspace_bytes", "dsa_indexer_scores",
            "dsa_indexer_topk_varlen_workspace_bytes", "dsa_indexer_topk_varlen",
            "dsa_sparse_prefill_varlen_workspace_bytes", "dsa_sparse_prefill_varlen",
            "dsa_retrieval_topk_workspace_bytes", "dsa_retrieval_topk",
            "dsa_sparse_prefill_gate", "dsa_ceiling_mfma_threads", "dsa_ceiling_mfma_bf16",
            "dsa_ceiling_stream_sink_words", "dsa_ceiling_stream",
            "dsa_profile_enable", "dsa_profile_set",
            "dsa_profile_read", "dsa_status_string", "dsa_last_error", "dsa_version"]
PROFILE_KERNELS = ["key_stats", "score_sample", "row_prep", "score_filter", "select", "fold",
                   "sparse_attention", "causal_mask", "attn_split", "attn_merge", "retr_prep", "retr_sample",
                   "retr_filter", "retr_gather", "ceiling_mfma", "ceiling_copy"]

_lib = None


class IndexerStats(ctypes.Structure):
    """dsa_indexer_stats_t: selection counters of the last indexer call on a workspace."""
    _fields_ = [(n, ctypes.c_int64) for n in (
        "rows", "rows_all_keys", "rows_fallback", "fallback_overflow", "fallback_incomplete",
        "fallback_band", "rows_failed", "candidates", "candidates_max", "band", "band_max", "kth_radix")]


class DSAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")


def load_library(path: str | None = None):
    """Load libdsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    p = Path(path) if path else LIB_PATH
    if not p.exists():
        raise RuntimeError(f"{p} is missing: build it with `python -m dsa_sparse_attention_indexer_amd.build`")
    lib = ctypes.CDLL(str(p))
    P, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.dsa_indexer_topk_workspace_bytes.restype = sz
    lib.dsa_indexer_topk_workspace_bytes.argtypes = [i64, i64, i32, i32]
    lib.dsa_indexer_topk.restype = ctypes.c_int
    lib.dsa_indexer_topk.argtypes = [P, P, P, i64, i64, i32, i32, i64, i32, i32, P, P, sz, P]
    lib.dsa_indexer_key_cache_bytes.restype = sz
    lib.dsa_indexer_key_cache_bytes.argtypes = [i64]
    lib.dsa_indexer_key_cache_append.restype = ctypes.c_int
    lib.dsa_indexer_key_cache_append.argtypes = [P, i64, i64, P, sz, P]
    lib.dsa_indexer_topk_cached_workspace_bytes.restype = sz
    lib.dsa_indexer_topk_cached_workspace_bytes.argtypes = [i64, i64, i32, i32]
    lib.dsa_indexer_topk_cached.restype = ctypes.c_int
    lib.dsa_indexer_topk_cached.argtypes = [P, P, P, i64, i64, i32, i32, i64, i32, i32, P, P, sz, i64, P, sz, P]
    lib.dsa_indexer_topk_noalloc.restype = ctypes.c_int
    lib.dsa_indexer_topk_noalloc.argtypes = [P, P, P, i64, i64, i32, i32, i64, i32, i32, P, P]
    lib.dsa_indexer_topk_stats.restype = ctypes.c_int
    lib.dsa_indexer_topk_stats.argtypes = [P, P, P]
    lib.dsa_indexer_scores_workspace_bytes.restype = sz
    lib.dsa_indexer_scores_workspace_bytes.argtypes = [i64, i64]
    lib.dsa_indexer_scores.restype = ctypes.c_int
    lib.dsa_indexer_scores.argtypes = [P, P, P, i64, i64, i32, i32, i64, P, P, P, sz, P]
    lib.dsa_causal_mask_topk.restype = ctypes.c_int
    lib.dsa_causal_mask_topk.argtypes = [P, i64, i32, i64, P]
    lib.dsa_sparse_prefill.restype = ctypes.c_int
    lib.dsa_sparse_prefill.argtypes = [P, P, i64, P, i64, i64, i32, i32, i32, i32, i64, f32, i32, P, P, P]
    lib.dsa_sparse_prefill_packed.restype = ctypes.c_int
    lib.dsa_sparse_prefill_packed.argtypes = lib.dsa_sparse_prefill.argtypes
    lib.dsa_sparse_decode_workspace_bytes.restype = sz
    lib.dsa_sparse_decode_workspace_bytes.argtypes = [i64, i32, i32, i32]
    lib.dsa_sparse_decode.restype = ctypes.c_int
    lib.dsa_sparse_decode.argtypes = [P, P, i64, P, i64, i64, i32, i32, i32, i32, i64, f32, i32, P, P, P, sz, P]
    lib.dsa_indexer_topk_varlen_workspace_bytes.restype = sz
    lib.dsa_indexer_topk_varlen_workspace_bytes.argtypes = [i64, P, P, P, i32, i32]
    lib.dsa_indexer_topk_varlen.restype = ctypes.c_int
    lib.dsa_indexer_topk_varlen.argtypes = [P, P, P, i64, P, P, P, i32, i32, i32, i32, P, P, sz, P]
    lib.dsa_sparse_prefill_varlen_workspace_bytes.restype = sz
    lib.dsa_sparse_prefill_varlen_workspace_bytes.argtypes = [i64, P, P, P, i32, i32, i32]
    lib.dsa_sparse_prefill_varlen.restype = ctypes.c_int
    lib.dsa_sparse_prefill_varlen.argtypes = [P, P, i64, P, i64, P, P, P, i32, i32, i32, i32, f32, i32, P, P,
                                              P, sz, P]
    lib.dsa_retrieval_topk_workspace_bytes.restype = sz
    lib.dsa_retrieval_topk_workspace_bytes.argtypes = [i64, i64, i32, i32]
    lib.dsa_retrieval_topk.restype = ctypes.c_int
    lib.dsa_retrieval_topk.argtypes = [P, P, i64, i64, i32, i32, i32, P, P, sz, P]
    lib.dsa_sparse_prefill_gate.restype = ctypes.c_int
    lib.dsa_sparse_prefill_gate.argtypes = [i64, i64, i64, i64]
    lib.dsa_ceiling_mfma_threads.restype = i64
    lib.dsa_ceiling_mfma_threads.argtypes = [ctypes.c_int32]
    lib.dsa_ceiling_mfma_bf16.restype = ctypes.c_int
    lib.dsa_ceiling_mfma_bf16.argtypes = [ctypes.c_void_p, i64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    lib.dsa_ceiling_stream_sink_words.restype = i64
    lib.dsa_ceiling_stream_sink_words.argtypes = []
    lib.dsa_ceiling_stream.restype = ctypes.c_int
    lib.dsa_ceiling_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, i64,
                                       ctypes.c_int32, ctypes.c_void_p]
    lib.dsa_status_string.restype = ctypes.c_char_p
    lib.dsa_status_string.argtypes = [ctypes.c_int]
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_last_error.argtypes = []
    lib.dsa_version.restype = ctypes.c_char_p
    lib.dsa_version.argtypes = []
    lib.dsa_profile_enable.restype = ctypes.c_int
    lib.dsa_profile_enable.argtypes = [ctypes.c_int]
    lib.dsa_profile_set.restype = ctypes.c_int
    lib.dsa_profile_set.argtypes = [ctypes.c_char_p]
    lib.dsa_profile_read.restype = ctypes.c_int
    lib.dsa_profile_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int64)]
    _lib = lib
    return lib


def _check(status: int):
    if status != DSA_OK:
        raise DSAError(status, _lib.dsa_last_error().decode())


def _stream_ptr(tensor, stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(tensor.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _req(t, name, dtype, ndim):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got shape {tuple(t.shape)})")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def version() -> str:
    return load_library().dsa_version().decode()


def profile_enable(on: bool = True):
    """Bracket every library kernel launch with HIP events on its stream."""
    _check(load_library().dsa_profile_enable(1 if on else 0))


def profile_set(kernels=None):
    """Bracket only the given kernel classes (iterable of names; None = all) and turn timing on."""
    names = "" if kernels is None else ",".join(kernels)
    _check(load_library().dsa_profile_set(names.encode()))


def profile_read(kernel: str):
    """(total_ms, launches) of one kernel class since its last read; waits for its events."""
    lib = load_library()
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(lib.dsa_profile_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def workspace_bytes(L: int, N: int, top_k: int, q_block: int = DEFAULT_Q_BLOCK) -> int:
    return int(load_library().dsa_indexer_topk_workspace_bytes(L, N, top_k, q_block))


def sparse_prefill_gate(B: int, L: int, N: int, min_context: int = 16384) -> bool:
    return bool(load_library().dsa_sparse_prefill_gate(B, L, N, min_context))


def ceiling_mfma(out, iters: int, random_operands: bool, waves_per_simd: int = 1, stream=None) -> float:
    """Enqueue the MFMA-only ceiling loop (dsa_ceiling_mfma_bf16) writing to the fp32 GPU tensor
    out (at least ceiling_mfma_threads(waves_per_simd) elements); returns the launch's flops."""
    import torch

    lib = load_library()
    if not (isinstance(out, torch.Tensor) and out.is_cuda and out.dtype == torch.float32 and out.is_contiguous()):
        raise ValueError("out must be a contiguous fp32 GPU tensor")
    flops = ctypes.c_double()
    _check(lib.dsa_ceiling_mfma_bf16(out.data_ptr(), out.numel(), iters, 1 if random_operands else 0,
                                     waves_per_simd, ctypes.byref(flops), _stream_ptr(out, stream)))
    return flops.value


def ceiling_mfma_threads(waves_per_simd: int = 1) -> int:
    return int(load_library().dsa_ceiling_mfma_threads(waves_per_simd))


def ceiling_stream(src, dst=None, sink=None, nontemporal: bool = False, stream=None):
    """Enqueue the streaming ceiling (dsa_ceiling_stream): a copy of src into dst (same byte size),
    or with dst None a read of src whose per-thread XORs go to sink (int32 GPU tensor of at least
    ceiling_stream_sink_words() elements)."""
    import torch

    lib = load_library()
    for t, n in ((src, "src"), (dst, "dst"), (sink, "sink")):
        if t is not None and not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{n} must be a contiguous GPU tensor")
    nbytes = src.numel() * src.element_size()
    if dst is not None and dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same byte size")
    _check(lib.dsa_ceiling_stream(src.data_ptr(), dst.data_ptr() if dst is not None else None, nbytes,
                                  sink.data_ptr() if sink is not None else None,
                                  sink.numel() if sink is not None else 0, 1 if nontemporal else 0,
                                  _stream_ptr(src, stream)))


def ceiling_stream_sink_words() -> int:
    return int(load_library().dsa_ceiling_stream_sink_words())


def indexer_topk(q_idx, k_idx, w, q_pos0: int, top_k: int, q_block: int = DEFAULT_Q_BLOCK,
                 out=None, workspace=None, stream=None):
    """Exact top-k key indices per query (ascending, -1 padded) -> int32 [L, top_k].

    q_idx bf16 [L, 32, 128]; k_idx bf16 [N, 128]; w fp32 [L, 32]; query t sits at
    position q_pos0 + t and may select keys 0..q_pos0+t.
    """
    import torch

    lib = load_library()
    _req(q_idx, "q_idx", torch.bfloat16, 3)
    _req(k_idx, "k_idx", torch.bfloat16, 2)
    _req(w, "w", torch.float32, 2)
    L, nh, hd = q_idx.shape
    N = k_idx.shape[0]
    dev = q_idx.device
    if out is None:
        out = torch.empty((L, top_k), dtype=torch.int32, device=dev)
    else:
        _req(out, "out", torch.int32, 2)
    need = lib.dsa_indexer_topk_workspace_bytes(L, N, top_k, q_block)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    _check(lib.dsa_indexer_topk(q_idx.data_ptr(), k_idx.data_ptr(), w.data_ptr(), L, N, nh, hd,
                                q_pos0, top_k, q_block, out.data_ptr(), workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), _stream_ptr(q_idx, stream)))
    return out


def indexer_stats(workspace, stream=None) -> dict:
    """Selection counters of the last indexer / retrieval call made with `workspace` (a
    uint8 device tensor).  Waits for the stream."""
    lib = load_library()
    st = IndexerStats()
    _check(lib.dsa_indexer_topk_stats(workspace.data_ptr(), ctypes.byref(st), _stream_ptr(workspace, stream)))
    return {name: int(getattr(st, name)) for name, _ in IndexerStats._fields_}


def indexer_scores(q_idx, k_idx, w, q_pos0: int, stream=None):
    """Diagnostic: the fp32 scores the indexer's scoring kernel computes for every causal key of
    up to 64 query rows, and the rows' error bounds delta.  -> (fp32 [L, N] with NaN after each
    row's position, fp32 [L])."""
    import torch

    lib = load_library()
    _req(q_idx, "q_idx", torch.bfloat16, 3)
    _req(k_idx, "k_idx", torch.bfloat16, 2)
    _req(w, "w", torch.float32, 2)
    L, nh, hd = q_idx.shape
    N = k_idx.shape[0]
    dev = q_idx.device
    scores = torch.empty((L, N), dtype=torch.float32, device=dev)
    delta = torch.empty((L,), dtype=torch.float32, device=dev)
    need = int(lib.dsa_indexer_scores_workspace_bytes(L, N))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib.dsa_indexer_scores(q_idx.data_ptr(), k_idx.data_ptr(), w.data_ptr(), L, N, nh, hd, q_pos0,
                                  scores.data_ptr(), delta.data_ptr(), ws.data_ptr(), ws.numel(),
                                  _stream_ptr(q_idx, stream)))
    return scores, delta


class KeyCache:
    """An append-only indexer key cache on a GPU (dsa_indexer_key_cache_*): holds the tiled
    layout and error-bound statistics of up to `capacity` keys."""

    def __init__(self, capacity: int, device="cuda:0"):
        import torch

        lib = load_library()
        n = int(lib.dsa_indexer_key_cache_bytes(capacity))
        if n == 0:
            raise ValueError(f"bad key cache capacity {capacity}")
        self.capacity = capacity
        self.buffer = torch.empty(n, dtype=torch.uint8, device=device)
        self.n = 0

    def append(self, k_idx, n_new: int | None = None, stream=None):
        """Append rows self.n .. n_new-1 of k_idx (bf16 [>= n_new, 128]); n_new defaults to all rows."""
        import torch

        _req(k_idx, "k_idx", torch.bfloat16, 2)
        n_new = k_idx.shape[0] if n_new is None else n_new
        _check(load_library().dsa_indexer_key_cache_append(k_idx.data_ptr(), self.n, n_new, self.buffer.data_ptr(),
                                                           self.buffer.numel(), _stream_ptr(k_idx, stream)))
        self.n = n_new

    def reset(self):
        self.n = 0


def cached_workspace_bytes(L: int, N: int, top_k: int, q_block: int = DEFAULT_Q_BLOCK) -> int:
    return int(load_library().dsa_indexer_topk_cached_workspace_bytes(L, N, top_k, q_block))


def indexer_topk_cached(q_idx, k_idx, w, q_pos0: int, top_k: int, cache: "KeyCache",
                        q_block: int = DEFAULT_Q_BLOCK, out=None, workspace=None, stream=None):
    """indexer_topk with the keys' layout and statistics from a KeyCache holding cache.n keys."""
    import torch

    lib = load_library()
    _req(q_idx, "q_idx", torch.bfloat16, 3)
    _req(k_idx, "k_idx", torch.bfloat16, 2)
    _req(w, "w", torch.float32, 2)
    L, nh, hd = q_idx.shape
    N = k_idx.shape[0]
    dev = q_idx.device
    if out is None:
        out = torch.empty((L, top_k), dtype=torch.int32, device=dev)
    else:
        _req(out, "out", torch.int32, 2)
    if workspace is None:
        need = lib.dsa_indexer_topk_cached_workspace_bytes(L, N, top_k, q_block)
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    _check(lib.dsa_indexer_topk_cached(q_idx.data_ptr(), k_idx.data_ptr(), w.data_ptr(), L, N, nh, hd, q_pos0,
                                       top_k, q_block, out.data_ptr(), cache.buffer.data_ptr(),
                                       cache.buffer.numel(), cache.n, workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(), _stream_ptr(q_idx, stream)))
    return out


def causal_mask_topk(idx, q_pos0: int, stream=None):
    """In place: idx[t, j] > q_pos0 + t becomes -1.  Returns idx."""
    import torch

    lib = load_library()
    _req(idx, "idx", torch.int32, 2)
    L, k = idx.shape
    _check(lib.dsa_causal_mask_topk(idx.data_ptr(), L, k, q_pos0, _stream_ptr(idx, stream)))
    return idx


def sparse_prefill(q, kv, idx, q_pos0: int, scale: float, q_block: int = DEFAULT_Q_BLOCK,
                   return_lse: bool = False, out=None, lse=None, stream=None, pack: bool = False):
    """Sparse absorbed-MLA attention -> bf16 [L, H, 512] (and fp32 lse [L, H]).

    q bf16 [L, H, 576]; kv bf16 [N, >=576] (latent 0..511 | rope 512..575, the
    latent is also the value); idx int32 [L, top_k] (-1 and future keys skipped).
    pack=True gathers the union of neighbouring queries' rows once (same result up to
    the rounding order of the softmax sums); on MI355X it is slower than the default at
    every overlap measured (0.59x-0.96x).
    """
    import torch

    lib = load_library()
    _req(q, "q", torch.bfloat16, 3)
    _req(idx, "idx", torch.int32, 2)
    if not (isinstance(kv, torch.Tensor) and kv.dtype == torch.bfloat16 and kv.dim() == 2 and kv.is_cuda
            and kv.stride(1) == 1):
        raise ValueError("kv must be a bf16 GPU tensor [N, stride>=576] with unit column stride")
    L, H, dqk = q.shape
    N = kv.shape[0]
    top_k = idx.shape[1]
    if dqk != D_LATENT + D_ROPE:
        raise ValueError(f"q must be [L, H, {D_LATENT + D_ROPE}]")
    if idx.shape[0] != L:
        raise ValueError("idx must have L rows")
    if out is None:
        out = torch.empty((L, H, D_LATENT), dtype=torch.bfloat16, device=q.device)
    else:
        _req(out, "out", torch.bfloat16, 3)
    if return_lse and lse is None:
        lse = torch.empty((L, H), dtype=torch.float32, device=q.device)
    fn = lib.dsa_sparse_prefill_packed if pack else lib.dsa_sparse_prefill
    _check(fn(q.data_ptr(), kv.data_ptr(), kv.stride(0), idx.data_ptr(), L, N, H,
              D_LATENT, D_ROPE, top_k, q_pos0, float(scale), q_block, out.data_ptr(),
              lse.data_ptr() if lse is not None else None, _stream_ptr(q, stream)))
    return (out, lse) if return_lse else out


def decode_workspace_bytes(L: int, H: int, top_k: int, splits: int = 0) -> int:
    return int(load_library().dsa_sparse_decode_workspace_bytes(L, H, top_k, splits))


def sparse_decode(q, kv, idx, q_pos0: int, scale: float, splits: int = 0, return_lse: bool = False,
                  out=None, lse=None, workspace=None, stream=None):
    """Split-key sparse attention (decode and short chunks): the sparse_prefill result,
    with each query's top-k list cut into `splits` parts merged by log-sum-exp.

    Arguments as sparse_prefill; splits = 0 picks the count.  workspace: optional uint8
    GPU tensor of at least decode_workspace_bytes(L, H, top_k, splits) bytes.
    """
    import torch

    lib = load_library()
    _req(q, "q", torch.bfloat16, 3)
    _req(idx, "idx", torch.int32, 2)
    if not (isinstance(kv, torch.Tensor) and kv.dtype == torch.bfloat16 and kv.dim() == 2 and kv.is_cuda
            and kv.stride(1) == 1):
        raise ValueError("kv must be a bf16 GPU tensor [N, stride>=576] with unit column stride")
    L, H, dqk = q.shape
    N = kv.shape[0]
    top_k = idx.shape[1]
    if dqk != D_LATENT + D_ROPE:
        raise ValueError(f"q must be [L, H, {D_LATENT + D_ROPE}]")
    if idx.shape[0] != L:
        raise ValueError("idx must have L rows")
    if out is None:
        out = torch.empty((L, H, D_LATENT), dtype=torch.bfloat16, device=q.device)
    else:
        _req(out, "out", torch.bfloat16, 3)
    if return_lse and lse is None:
        lse = torch.empty((L, H), dtype=torch.float32, device=q.device)
    need = max(decode_workspace_bytes(L, H, top_k, splits), 1)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib.dsa_sparse_decode(q.data_ptr(), kv.data_ptr(), kv.stride(0), idx.data_ptr(), L, N, H,
                                 D_LATENT, D_ROPE, top_k, q_pos0, float(scale), splits, out.data_ptr(),
                                 lse.data_ptr() if lse is not None else None, workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), _stream_ptr(q, stream)))
    return (out, lse) if return_lse else out


def _host_i64(x, name, n):
    """A host int64 array of n entries (list, tuple, numpy array or CPU tensor)."""
    vals = [int(v) for v in (x.tolist() if hasattr(x, "tolist") else x)]
    if len(vals) != n:
        raise ValueError(f"{name} must have {n} entries (got {len(vals)})")
    return (ctypes.c_int64 * max(n, 1))(*vals)


def _batch(cu_q, cu_k, pos0):
    B = len(pos0.tolist() if hasattr(pos0, "tolist") else pos0)
    return B, _host_i64(cu_q, "cu_q", B + 1), _host_i64(cu_k, "cu_k", B + 1), _host_i64(pos0, "pos0", B)


def varlen_workspace_bytes(cu_q, cu_k, pos0, top_k: int, q_block: int = DEFAULT_Q_BLOCK) -> int:
    B, cq, ck, p0 = _batch(cu_q, cu_k, pos0)
    return int(load_library().dsa_indexer_topk_varlen_workspace_bytes(B, cq, ck, p0, top_k, q_block))


def indexer_topk_varlen(q_idx, k_idx, w, cu_q, cu_k, pos0, top_k: int, q_block: int = DEFAULT_Q_BLOCK,
                        out=None, workspace=None, stream=None):
    """indexer_topk for each sequence of a packed batch -> int32 [T, top_k].

    Sequence b owns query rows cu_q[b]..cu_q[b+1]-1 of q_idx [T, 32, 128] and w [T, 32],
    keys cu_k[b]..cu_k[b+1]-1 of k_idx, and its first query sits at position pos0[b].
    Indices are positions within the sequence.  cu_q, cu_k, pos0 live on the host.
    """
    import torch

    lib = load_library()
    _req(q_idx, "q_idx", torch.bfloat16, 3)
    _req(k_idx, "k_idx", torch.bfloat16, 2)
    _req(w, "w", torch.float32, 2)
    B, cq, ck, p0 = _batch(cu_q, cu_k, pos0)
    T, nh, hd = q_idx.shape
    if B > 0 and (cq[B] != T or ck[B] > k_idx.shape[0] or w.shape[0] != T):
        raise ValueError("cu_q[B] must equal the query rows and cu_k[B] fit k_idx")
    dev = q_idx.device
    if out is None:
        out = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    else:
        _req(out, "out", torch.int32, 2)
    need = lib.dsa_indexer_topk_varlen_workspace_bytes(B, cq, ck, p0, top_k, q_block)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    _check(lib.dsa_indexer_topk_varlen(q_idx.data_ptr(), k_idx.data_ptr(), w.data_ptr(), B, cq, ck, p0, nh, hd,
                                       top_k, q_block, out.data_ptr(), workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(), _stream_ptr(q_idx, stream)))
    return out


def prefill_varlen_workspace_bytes(cu_q, cu_k, pos0, H: int, top_k: int, splits: int = 1) -> int:
    B, cq, ck, p0 = _batch(cu_q, cu_k, pos0)
    return int(load_library().dsa_sparse_prefill_varlen_workspace_bytes(B, cq, ck, p0, H, top_k, splits))


def sparse_prefill_varlen(q, kv, idx, cu_q, cu_k, pos0, scale: float, splits: int = 1, return_lse: bool = False,
                          out=None, lse=None, workspace=None, stream=None):
    """sparse_prefill for each sequence of a packed batch -> bf16 [T, H, 512] (and lse).

    q [T, H, 576], idx [T, top_k] (positions within each sequence), kv rows
    cu_k[b]..cu_k[b+1]-1 belong to sequence b.  splits as sparse_decode (1: one
    workgroup per query; 0: picked from T).
    """
    import torch

    lib = load_library()
    _req(q, "q", torch.bfloat16, 3)
    _req(idx, "idx", torch.int32, 2)
    if not (isinstance(kv, torch.Tensor) and kv.dtype == torch.bfloat16 and kv.dim() == 2 and kv.is_cuda
            and kv.stride(1) == 1):
        raise ValueError("kv must be a bf16 GPU tensor [N, stride>=576] with unit column stride")
    B, cq, ck, p0 = _batch(cu_q, cu_k, pos0)
    T, H, dqk = q.shape
    top_k = idx.shape[1]
    if dqk != D_LATENT + D_ROPE:
        raise ValueError(f"q must be [T, H, {D_LATENT + D_ROPE}]")
    if idx.shape[0] != T or (B > 0 and (cq[B] != T or ck[B] > kv.shape[0])):
        raise ValueError("idx must have T rows, cu_q[B] must equal T and cu_k[B] fit kv")
    if out is None:
        out = torch.empty((T, H, D_LATENT), dtype=torch.bfloat16, device=q.device)
    else:
        _req(out, "out", torch.bfloat16, 3)
    if return_lse and lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    need = lib.dsa_sparse_prefill_varlen_workspace_bytes(B, cq, ck, p0, H, top_k, splits)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=q.device)
    _check(lib.dsa_sparse_prefill_varlen(q.data_ptr(), kv.data_ptr(), kv.stride(0), idx.data_ptr(), B, cq, ck, p0,
                                         H, D_LATENT, D_ROPE, top_k, float(scale), splits, out.data_ptr(),
                                         lse.data_ptr() if lse is not None else None, workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(), _stream_ptr(q, stream)))
    return (out, lse) if return_lse else out


def retrieval_workspace_bytes(M: int, N: int, top_k: int, q_block: int = DEFAULT_Q_BLOCK) -> int:
    return int(load_library().dsa_retrieval_topk_workspace_bytes(M, N, top_k, q_block))


def retrieval_topk(q, x, top_k: int, q_block: int = DEFAULT_Q_BLOCK, out=None, workspace=None, stream=None):
    """Exact inner-product top-k corpus rows per query (ascending, -1 padded) -> int32 [M, top_k].

    q bf16 [M, 128] queries; x bf16 [N, 128] corpus.  Ranked by q . x (fp64 left-to-right
    order), lower row first among equal scores.
    """
    import torch

    lib = load_library()
    _req(q, "q", torch.bfloat16, 2)
    _req(x, "x", torch.bfloat16, 2)
    M, d = q.shape
    N = x.shape[0]
    if x.shape[1] != d:
        raise ValueError("q and x must have the same row width")
    if out is None:
        out = torch.empty((M, top_k), dtype=torch.int32, device=q.device)
    else:
        _req(out, "out", torch.int32, 2)
    need = lib.dsa_retrieval_topk_workspace_bytes(M, N, top_k, q_block)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=q.device)
    _check(lib.dsa_retrieval_topk(q.data_ptr(), x.data_ptr(), M, N, d, top_k, q_block, out.data_ptr(),
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  _stream_ptr(q, stream)))
    return out
