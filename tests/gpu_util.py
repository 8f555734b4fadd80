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


def _max(a: float, b: float) -> float:
    """max that keeps a NaN (Python's max drops one in the second place)."""
    return a if (a != a or a >= b) else b


class Parity:
    """Errors of a GPU result against the oracle, accumulated over blocks that each
    hold whole rows (a row is the reduced axis: (b, d) over t for a scan's out,
    over steps for decode, over n for a state).

      row_inf    max over rows of max|y - ref| / max|ref| (the gated metric);
      elem_rms   max over elements of |y - ref| / max(|ref|, rms of the row);
      elem_rms3  the same with the floor 1e-3 * rms of the row;
      whole_inf  max|y - ref| / max|ref| over the whole tensor.
    NaN anywhere in the error makes every metric NaN, so a bar check fails."""

    def __init__(self, name: str):
        self.name = name
        self.row_inf = 0.0
        self.elem_rms = 0.0
        self.elem_rms3 = 0.0
        self.max_err = 0.0
        self.max_ref = 0.0
        self.count = 0

    def add(self, y, ref, axis):
        y = np.asarray(y, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert y.shape == ref.shape, (y.shape, ref.shape)
        if y.size == 0:
            return self
        err = np.abs(y - ref)
        aref = np.abs(ref)
        den = np.max(aref, axis=axis, keepdims=True)
        self.row_inf = _max(self.row_inf, float(np.max(np.max(err, axis=axis, keepdims=True) /
                                                       np.where(den > 0, den, 1.0))))
        rms = np.sqrt(np.mean(ref * ref, axis=axis, keepdims=True))
        for attr, floor in (("elem_rms", rms), ("elem_rms3", 1e-3 * rms)):
            f = np.maximum(aref, floor)
            setattr(self, attr, _max(getattr(self, attr), float(np.max(err / np.where(f > 0, f, 1.0)))))
        self.max_err = _max(self.max_err, float(np.max(err)))
        self.max_ref = _max(self.max_ref, float(np.max(aref)))
        self.count += y.size
        return self

    @property
    def whole_inf(self) -> float:
        return self.max_err / self.max_ref if self.max_ref > 0 else self.max_err

    def report(self) -> str:
        return (f"{self.name}: {self.count} values, row_inf {self.row_inf:.3e}, elem_rms {self.elem_rms:.3e}, "
                f"elem_rms3 {self.elem_rms3:.3e}, whole_inf {self.whole_inf:.3e}")

    def check(self, gate: float, tight: float | None = None, tight_rms3: float | None = None):
        """Gate: row_inf and elem_rms <= gate.  tight: every metric but elem_rms3 <= tight
        (inputs are identical on both sides, so only fp32 rounding differs); tight_rms3:
        elem_rms3 <= tight_rms3."""
        print(f"[parity] {self.report()}", flush=True)
        assert self.count > 0, self.name
        assert self.row_inf <= gate, self.report()
        assert self.elem_rms <= gate, self.report()
        if tight is not None:
            assert max(self.row_inf, self.elem_rms, self.whole_inf) <= tight, self.report()
        if tight_rms3 is not None:
            assert self.elem_rms3 <= tight_rms3, self.report()
