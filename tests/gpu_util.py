"""Helpers for the GPU parity tests: numpy <-> torch device tensors and the
attention tolerance check.  No method arithmetic lives here."""
import functools

import numpy as np

# Attention tolerance on bf16 outputs: max |gpu - oracle| and relative L2 error of the
# whole compared tensor.
ATTN_MAX_ABS = 2e-2
ATTN_REL_L2 = 5e-3


def to_dev_bf16(bits: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def to_dev(arr: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(arr)).to("cuda:0")


def bf16_dev_to_f64(t) -> np.ndarray:
    import torch

    return t.float().cpu().numpy().astype(np.float64)


def bits_of(t) -> np.ndarray:
    import torch

    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def attn_errors(gpu: np.ndarray, ref: np.ndarray):
    diff = gpu - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / den if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_attn_close(gpu: np.ndarray, ref: np.ndarray, what: str = ""):
    max_abs, rel = attn_errors(gpu, ref)
    assert max_abs <= ATTN_MAX_ABS and rel <= ATTN_REL_L2, f"{what}: max_abs={max_abs:.3g} rel_l2={rel:.3g}"
    return max_abs, rel


def report(msg: str):
    print(msg, flush=True)


@functools.lru_cache(maxsize=3)
def config_inputs(name: str):
    """make_inputs of a named configuration or integer twin ("C3", "C4i"), kept for reuse
    across tests (C4's draws take seconds)."""
    import dsa_inputs as di

    wl = di.int_twin(name[:2]) if name.endswith("i") else di.CONFIGS[name]
    return wl, di.make_inputs(wl)
