"""Shared helpers for the GPU tests: upload synthetic inputs, compare against the oracle."""
from __future__ import annotations

import numpy as np
import torch


def bits_to_torch(bits: np.ndarray, dtype: torch.dtype, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(dtype).to(device)


def upload(x: dict, device="cuda") -> dict:
    """synth.make_config output -> device tensors with the library's dtypes."""
    q = x["q"]
    d = {
        "q": bits_to_torch(q, torch.bfloat16, device) if q.dtype == np.uint16 else torch.from_numpy(q).to(device),
        "pos": torch.from_numpy(np.ascontiguousarray(x["pos"], dtype=np.int64)).to(device),
        "raw": bits_to_torch(x["raw"], torch.float16, device),
        "comp": bits_to_torch(x["comp"], torch.bfloat16, device),
        "idx_k": bits_to_torch(x["idx_k"], torch.bfloat16, device),
        "idx_q": bits_to_torch(x["idx_q"], torch.bfloat16, device),
        "idx_w": torch.from_numpy(np.ascontiguousarray(x["idx_w"], dtype=np.float32)).to(device),
        "n_vis": torch.from_numpy(np.ascontiguousarray(x["n_vis"], dtype=np.int32)).to(device),
    }
    return d


def normwise_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| over one (unit, query)'s H x D outputs."""
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(got.astype(np.float64) - ref)))
    return num / den if den > 0 else num


def tie_band_ok(gpu_set: np.ndarray, ref_rank: np.ndarray, ref_scores: np.ndarray, rel: float = 1e-5):
    """Selected sets may differ only in rows whose oracle score lies within rel of the oracle's
    K-th score.  Returns (ok, number of differing rows)."""
    ref_set = ref_rank[ref_rank >= 0]
    g = set(int(j) for j in gpu_set if j >= 0)
    r = set(int(j) for j in ref_set)
    diff = g ^ r
    if not diff:
        return True, 0
    if len(g) != len(r):
        return False, len(diff)
    kth = float(ref_scores[ref_set[-1]])
    band = rel * abs(kth)
    return all(abs(float(ref_scores[j]) - kth) <= band for j in diff), len(diff)
