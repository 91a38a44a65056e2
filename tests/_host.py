"""Host-side helpers shared by the tests: move tensors to numpy in the form the oracle reads, and build small
seeded paged batches on the CPU."""

from __future__ import annotations

import numpy as np
import torch

from workloads import custom_structure, materialize


def to_host(t: torch.Tensor) -> np.ndarray:
    """float32 tensors become float32 arrays; bfloat16 tensors uint16 arrays of their bit patterns; float8_e4m3fn
    tensors uint8 arrays of their codes."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy().copy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy().copy()
    if t.dtype == torch.int32:
        return t.numpy().copy()
    raise TypeError(t.dtype)


def small_case(seed, lens, hq, hkv, d, bs, dtype, include_new_token=True, **kw):
    """A seeded paged batch on the CPU: (structure, dict of host arrays)."""
    st = custom_structure(f"small{seed}", seed, lens, hq, hkv, d, bs, dtype, **kw)
    tensors = materialize(st, "cpu", include_new_token=include_new_token)
    return st, {k: to_host(v) for k, v in tensors.items()}


def f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)
