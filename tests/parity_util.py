"""Helpers of the GPU parity tests: host <-> device copies and comparisons.

Nothing here computes a collective: the expected side always comes from
``oracle`` and the tested side from the HIP library.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}
NP_DTYPE = {"f32": np.float32, "bf16": np.uint16, "i32": np.int32}


def say(*a):
    """Name the case before a GPU step, flushed, so a crash still shows it."""
    print(*a, file=sys.stderr, flush=True)


def to_dev(x: np.ndarray, dtype: str, device="cuda:0") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x, np.uint16).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, NP_DTYPE[dtype])).to(device)


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def empty(n: int, dtype: str, device="cuda:0", fill=None) -> torch.Tensor:
    t = torch.empty(n, dtype=TORCH_DTYPE[dtype], device=device)
    if fill is not None:
        t.view(torch.int16 if dtype == "bf16" else t.dtype).fill_(fill)
    return t


def _bf16_ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def assert_parity(got: np.ndarray, want: np.ndarray, dtype: str, what: str = "") -> dict:
    """fp32 / int32: bit-exact.  bf16: at most 1 bf16 ulp apart, NaN where NaN.

    Returns {"n": elements, "exact": bit-identical elements, "max_ulp": ...}.
    """
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if dtype in ("f32", "i32"):
        g = got.view(np.uint32)
        w = want.view(np.uint32)
        bad = np.flatnonzero(g != w)
        if dtype == "f32":  # NaN payloads are not pinned: any NaN matches any NaN
            bad = bad[~(np.isnan(got[bad]) & np.isnan(want[bad]))]
        assert bad.size == 0, (
            f"{what}: {bad.size} of {got.size} differ; first at {bad[:5].tolist()}: "
            f"got {got[bad[:5]].tolist()} want {want[bad[:5]].tolist()}")
        return {"n": got.size, "exact": got.size, "max_ulp": 0}
    g = got.view(np.uint16)
    w = want.view(np.uint16)
    gn = (g & 0x7FFF) > 0x7F80
    wn = (w & 0x7FFF) > 0x7F80
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    ok = ~gn
    d = np.abs(_bf16_ordered(g[ok]) - _bf16_ordered(w[ok]))
    mx = int(d.max()) if d.size else 0
    assert mx <= 1, f"{what}: max bf16 ulp distance {mx} at {np.flatnonzero(ok)[np.argmax(d)]}"
    return {"n": got.size, "exact": int((g == w).sum()), "max_ulp": mx}
