"""Helpers of the GPU parity tests: host <-> device copies and comparisons.

Nothing here computes a collective: the expected side always comes from
``oracle`` and the tested side from the HIP library.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32,
               "f64": torch.float64, "f16": torch.float16, "i64": torch.int64,
               "u64": torch.uint64, "i8": torch.int8, "f32h": torch.float32}
NP_DTYPE = {"f32": np.float32, "bf16": np.uint16, "i32": np.int32, "f64": np.float64,
            "f16": np.uint16, "i64": np.int64, "u64": np.uint64, "i8": np.int8,
            "f32h": np.float32}
# a signed integer type of the same width, for filling and viewing raw bits
_BITS_T = {1: torch.int8, 2: torch.int16, 4: torch.int32, 8: torch.int64}
_BITS_NP = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}


def say(*a):
    """Name the case before a GPU step, flushed, so a crash still shows it."""
    print(*a, file=sys.stderr, flush=True)


def _width(dtype: str) -> int:
    return np.dtype(NP_DTYPE[dtype]).itemsize


def to_dev(x: np.ndarray, dtype: str, device="cuda:0") -> torch.Tensor:
    """Host array (bit patterns for bf16/f16) -> device tensor of the dtype, bit for bit."""
    w = _width(dtype)
    raw = np.ascontiguousarray(x, NP_DTYPE[dtype]).view(_BITS_NP[w]).view(np.dtype(f"i{w}"))
    return torch.from_numpy(raw).to(device).view(TORCH_DTYPE[dtype])


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Device tensor -> host array of NP_DTYPE (bit patterns for bf16/f16)."""
    w = _width(dtype)
    return t.view(_BITS_T[w]).cpu().numpy().view(NP_DTYPE[dtype])


def empty(n: int, dtype: str, device="cuda:0", fill=None) -> torch.Tensor:
    t = torch.empty(n, dtype=TORCH_DTYPE[dtype], device=device)
    if fill is not None:
        t.view(_BITS_T[_width(dtype)]).fill_(fill)
    return t


def _bf16_ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def assert_parity(got: np.ndarray, want: np.ndarray, dtype: str, what: str = "") -> dict:
    """Every type but bf16: bit-exact.  bf16: at most 1 bf16 ulp apart.  NaN where NaN.

    Returns {"n": elements, "exact": bit-identical elements, "max_ulp": ...}.
    """
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if dtype != "bf16":
        bits = _BITS_NP[_width(dtype)]
        g = got.view(bits)
        w = want.view(bits)
        bad = np.flatnonzero(g != w)
        if dtype in ("f32", "f64", "f16", "f32h"):  # NaN payloads are not pinned: any NaN matches any NaN
            gf = got.view(np.float16) if dtype == "f16" else got
            wf = want.view(np.float16) if dtype == "f16" else want
            bad = bad[~(np.isnan(gf[bad]) & np.isnan(wf[bad]))]
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
