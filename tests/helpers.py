"""Shared test helpers: tolerance check and numpy <-> torch transfers."""

from __future__ import annotations

import numpy as np
import torch


def tol_check(gpu: np.ndarray, ref32: np.ndarray, what: str, rms: float | None = None):
    """Per element: |gpu - oracle| <= 2^-7 |oracle| + 1e-3 rms(oracle), the
    floating-point parity bound of the FP8 and W4A16 GEMMs (oracle before its
    final bf16 rounding; rms over the whole output of the call unless given)."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref32, np.float64)
    if rms is None:
        rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    err = np.abs(g - r)
    bound = 2.0 ** -7 * np.abs(r) + 1e-3 * rms
    bad = err > bound
    if bad.any():
        i = np.flatnonzero(bad.ravel())[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{bad.size} outside tolerance; worst ratio "
            f"{float((err / np.maximum(bound, 1e-30)).max()):.3f}; first {i.tolist()}: gpu "
            f"{g.ravel()[i].tolist()} oracle {r.ravel()[i].tolist()}")
    return float((err / np.maximum(bound, 1e-30)).max()) if err.size else 0.0


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    """numpy -> device tensor (uint16 arrays become bfloat16 bit-for-bit)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    t = torch.from_numpy(a).cuda()
    return t if dtype is None else t.to(dtype)


def host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy (bfloat16 becomes uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)
