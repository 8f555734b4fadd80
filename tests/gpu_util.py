"""Helpers shared by the GPU parity tests (not a test module)."""
from __future__ import annotations

import sys

import numpy as np


def say(msg: str):
    """Name the case before a GPU step (flushed, so a failing box still shows it)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def rowinf(y, ref, axis) -> float:
    """Per-row infinity-norm relative error: max over rows of max|y - ref| / max|ref| along ``axis``."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    if y.size == 0:
        return 0.0
    num = np.max(np.abs(y - ref), axis=axis)
    den = np.max(np.abs(ref), axis=axis)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(num / den))


def to_dev(inp: dict, device="cuda"):
    """numpy inputs from ``workloads`` -> torch tensors on the GPU (bf16 where the config says so)."""
    import torch
    dt = inp.get("dtype", "f32")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = {}
    for k, v in inp.items():
        if k == "dtype":
            continue
        t = torch.from_numpy(np.ascontiguousarray(v))
        if k in ("x", "delta", "z", "B", "C"):
            t = t.to(tdt)  # exact: the values are representable in the input dtype
        out[k] = t.to(device)
    return out


def sample_channels(d_inner: int, n: int, seed: int = 0) -> np.ndarray:
    """Deterministic channel sample: the first and last channel, block edges, and random ones."""
    rng = np.random.default_rng(seed)
    pick = {0, d_inner - 1, min(63, d_inner - 1), min(64, d_inner - 1)}
    while len(pick) < min(n, d_inner):
        pick.add(int(rng.integers(0, d_inner)))
    return np.array(sorted(pick))


def slice_channels(inp: dict, sel: np.ndarray) -> dict:
    out = dict(inp)
    for k in ("x", "delta", "z"):
        out[k] = np.ascontiguousarray(inp[k][..., sel])
    out["A"] = np.ascontiguousarray(inp["A"][sel])
    out["D"] = np.ascontiguousarray(inp["D"][sel])
    out["delta_bias"] = np.ascontiguousarray(inp["delta_bias"][sel])
    return out


def rne_bf16_of(t):
    """Round a float32 torch tensor to bfloat16 (nearest even), returned as float32 on the CPU."""
    from workloads import round_to_bf16
    return round_to_bf16(t.float().cpu().numpy())
