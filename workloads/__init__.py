"""Seeded synthetic inputs for the selective scan and its decode step.

This module serves both the CPU oracle and the GPU library (tests and bench),
so it deliberately holds none of the scan's arithmetic: it only draws random
numbers, shapes them into tensors and rounds them to the input dtype.

Recipe (the same for every workload; the values come from the workload table):
  * A[d, n] = -exp(A_log[n]) with A_log[n] = log(n + 1), i.e. -(n + 1), fp32.
    (The Mamba-1 convention A = -exp(A_log), page "Mamba и State Space
    Models", Mamba-2 code block.)  ``random_params=True`` instead draws
    A[d, n] = -exp(U(-1, 3)), D ~ U(0.5, 1.5) and the bias per channel, so that
    per-channel indexing of A and D is exercised.
  * D[d] = 1 (random_params: U(0.5, 1.5)).
  * x, z, B, C ~ N(0, 1), drawn in float32.
  * The step size: a target Delta* ~ LogUniform[dmin, dmax] per (b, t, d) and a
    per-channel beta ~ LogUniform[dmin, dmax]; bias[d] = log(expm1(beta)) and
    delta = log(expm1(Delta*)) - bias[d].  Then softplus(delta + bias) gives
    back Delta* up to the rounding of delta to the input dtype.
  * The "DNA-like" long workload draws x[0, t, :] = W[tok_t, :] + 0.1 * eps with
    W ~ N(0, 1) of shape [4, d_inner], tok_t uniform on {0, 1, 2, 3} and
    eps ~ N(0, 1) (a four-letter alphabet of projected one-hot tokens).
  * Values are drawn in float32 (Delta* and beta in float64), then rounded
    to the input dtype: float32, or bfloat16 with round-to-nearest-even.  bf16
    tensors are returned as float32 arrays whose values are exactly
    representable in bf16; ``bf16_bits`` gives their 16-bit encodings.

Determinism: every tensor is split into blocks of rows; block i of tensor k
draws from PCG64(SeedSequence(seed, spawn_key=(k, i))).  The result does not
depend on the number of threads used to fill it.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "ScanConfig", "DecodeConfig", "SCAN_CONFIGS", "DECODE_CONFIG",
    "scan_inputs", "decode_inputs", "round_to_bf16", "bf16_bits",
    "scan_algorithmic_bytes", "decode_algorithmic_bytes",
    "SsdConfig", "SSD_CONFIGS", "ssd_inputs", "ssd_initial_state", "ssd_algorithmic_bytes",
]

# Tensor ids used as the first spawn key (stable; never renumber).
(_T_BIAS, _T_X, _T_DT, _T_Z, _T_B, _T_C, _T_W, _T_TOK, _T_BETA, _T_A, _T_D, _T_CW, _T_CB, _T_CS, _T_H0,
 _T_SA, _T_SD) = range(17)
_BLOCK_ELEMS = 1 << 20


@dataclasses.dataclass(frozen=True)
class ScanConfig:
    name: str
    batch: int
    d_inner: int
    d_state: int
    seqlen: int
    dtype: str            # "f32" or "bf16": dtype of x, delta, z, B, C
    dmin: float = 1e-3    # range of the softplus'ed step size
    dmax: float = 0.1
    x_kind: str = "normal"   # "normal" or "dna"
    description: str = ""


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    d_inner: int
    d_state: int
    steps: int
    dtype: str
    dmin: float = 1e-3
    dmax: float = 0.1
    description: str = ""


SCAN_CONFIGS = {
    "tiny_fp32": ScanConfig("tiny_fp32", 1, 64, 16, 256, "f32",
                            description="tiny scan, fp32 throughout"),
    "mamba130m": ScanConfig("mamba130m", 8, 1536, 16, 2048, "bf16",
                            description="Mamba-130M-like layer scan"),
    "mamba2p8b": ScanConfig("mamba2p8b", 8, 5120, 16, 2048, "bf16",
                            description="Mamba-2.8B-like layer scan"),
    "long_dna": ScanConfig("long_dna", 1, 2048, 16, 262144, "bf16", dmin=1e-4, x_kind="dna",
                           description="long-sequence DNA/audio-like scan"),
}


@dataclasses.dataclass(frozen=True)
class SsdConfig:
    """A Mamba-2 (SSD) layer: channels = nheads x headdim, B/C in ngroups groups."""
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    d_state: int
    dtype: str = "bf16"
    dmin: float = 1e-3
    dmax: float = 0.1
    description: str = ""


SSD_CONFIGS = {
    "mamba2_2p7b": SsdConfig("mamba2_2p7b", 8, 2048, 80, 64, 1, 128,
                             description="Mamba-2-2.7B-like SSD layer: 5120 channels as 80 heads x 64, "
                                         "d_state 128, one B/C group"),
}

DECODE_CONFIG = DecodeConfig("decode_b256", 256, 8192, 16, 512, "bf16",
                             description="decode state update, 512 steps at batch 256")


def _nthreads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _gen(seed: int, tensor: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor, block))))


def _fill(shape, seed: int, tensor: int, draw) -> np.ndarray:
    """Fill a float32 array of ``shape`` block by block; ``draw(gen, n)`` returns n values."""
    total = int(np.prod(shape, dtype=np.int64))
    out = np.empty(total, dtype=np.float32)
    nblk = max(1, -(-total // _BLOCK_ELEMS))

    def work(i):
        lo = i * _BLOCK_ELEMS
        hi = min(total, lo + _BLOCK_ELEMS)
        out[lo:hi] = draw(_gen(seed, tensor, i), hi - lo)

    if nblk == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_nthreads()) as ex:
            list(ex.map(work, range(nblk)))
    return out.reshape(shape)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    r = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    nan = np.isnan(a)
    if nan.any():
        r = np.where(nan, np.uint32(0x7FC00000), r)
    return r.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """16-bit encodings of float32 values that are exactly representable in bf16."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    if np.any(bits & np.uint32(0xFFFF)):
        raise ValueError("array holds values that are not bf16-representable")
    return (bits >> np.uint32(16)).astype(np.uint16)


def _to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16(a)
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal(shape, seed, tensor):
    return _fill(shape, seed, tensor, lambda g, n: g.standard_normal(n, dtype=np.float32))


def _log_uniform64(g: np.random.Generator, n: int, lo: float, hi: float) -> np.ndarray:
    u = g.random(n)
    return np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))


def _params(d_inner, d_state, dmin, dmax, seed, random_params):
    """A [d_inner, d_state], D [d_inner], delta_bias [d_inner] (all float32)."""
    if random_params:
        ga = _gen(seed, _T_A, 0)
        A = (-np.exp(ga.uniform(-1.0, 3.0, size=(d_inner, d_state)))).astype(np.float32)
        D = _gen(seed, _T_D, 0).uniform(0.5, 1.5, size=d_inner).astype(np.float32)
    else:
        a_log = np.log(np.arange(1, d_state + 1, dtype=np.float64))
        A = np.broadcast_to(-np.exp(a_log), (d_inner, d_state)).astype(np.float32)
        D = np.ones(d_inner, dtype=np.float32)
    beta = _log_uniform64(_gen(seed, _T_BETA, 0), d_inner, dmin, dmax)
    bias = np.log(np.expm1(beta)).astype(np.float32)
    return np.ascontiguousarray(A), D, bias


def _delta(shape, bias, dmin, dmax, seed, tensor):
    """delta[..., d] = log(expm1(Delta*)) - bias[d] with Delta* log-uniform (float32 result)."""
    d_inner = shape[-1]
    bias64 = bias.astype(np.float64)

    def draw(g, n):
        target = _log_uniform64(g, n, dmin, dmax)
        return np.log(np.expm1(target))

    raw = _fill(shape, seed, tensor, draw).reshape(-1, d_inner)
    return (raw.astype(np.float64) - bias64[None, :]).astype(np.float32).reshape(shape)


def scan_inputs(cfg: ScanConfig, seed: int = 0, random_params: bool = False,
                batch: int | None = None, seqlen: int | None = None, d_inner: int | None = None):
    """Inputs for ``ssm_scan_fwd`` under ``cfg`` (sizes may be overridden for small cases).

    Returns a dict of float32 numpy arrays: x, delta, z [batch, seqlen, d_inner];
    B, C [batch, seqlen, d_state]; A [d_inner, d_state]; D, delta_bias [d_inner];
    plus "dtype" (the input dtype name).
    """
    bsz = cfg.batch if batch is None else batch
    L = cfg.seqlen if seqlen is None else seqlen
    Dn = cfg.d_inner if d_inner is None else d_inner
    N = cfg.d_state
    A, D, bias = _params(Dn, N, cfg.dmin, cfg.dmax, seed, random_params)
    shape = (bsz, L, Dn)
    if cfg.x_kind == "dna":
        W = _normal((4, Dn), seed, _T_W)
        tok = _gen(seed, _T_TOK, 0).integers(0, 4, size=bsz * L)
        eps = _normal(shape, seed, _T_X).reshape(bsz * L, Dn)
        x = (W[tok] + np.float32(0.1) * eps).reshape(shape)
    else:
        x = _normal(shape, seed, _T_X)
    delta = _delta(shape, bias, cfg.dmin, cfg.dmax, seed, _T_DT)
    z = _normal(shape, seed, _T_Z)
    B = _normal((bsz, L, N), seed, _T_B)
    C = _normal((bsz, L, N), seed, _T_C)
    dt = cfg.dtype
    return {
        "x": _to_dtype(x, dt), "delta": _to_dtype(delta, dt), "z": _to_dtype(z, dt),
        "B": _to_dtype(B, dt), "C": _to_dtype(C, dt),
        "A": A, "D": D, "delta_bias": bias, "dtype": dt,
    }


def decode_inputs(cfg: DecodeConfig, seed: int = 0, steps: int | None = None,
                  batch: int | None = None, d_inner: int | None = None, random_params: bool = False):
    """Inputs for ``steps`` consecutive ``ssm_state_update`` calls.

    Returns a dict: x, delta, z [steps, batch, d_inner]; B, C [steps, batch, d_state];
    A, D, delta_bias as in ``scan_inputs``; "dtype".  Step s of a decode run is the
    time step s of a scan over the same tensors viewed as [batch, steps, ...].
    """
    S = cfg.steps if steps is None else steps
    bsz = cfg.batch if batch is None else batch
    Dn = cfg.d_inner if d_inner is None else d_inner
    N = cfg.d_state
    A, D, bias = _params(Dn, N, cfg.dmin, cfg.dmax, seed, random_params)
    shape = (S, bsz, Dn)
    x = _normal(shape, seed, _T_X)
    delta = _delta(shape, bias, cfg.dmin, cfg.dmax, seed, _T_DT)
    z = _normal(shape, seed, _T_Z)
    B = _normal((S, bsz, N), seed, _T_B)
    C = _normal((S, bsz, N), seed, _T_C)
    dt = cfg.dtype
    return {
        "x": _to_dtype(x, dt), "delta": _to_dtype(delta, dt), "z": _to_dtype(z, dt),
        "B": _to_dtype(B, dt), "C": _to_dtype(C, dt),
        "A": A, "D": D, "delta_bias": bias, "dtype": dt,
    }


def conv_inputs(batch: int, seqlen: int, d_inner: int, d_conv: int = 4, dtype: str = "bf16", seed: int = 0,
                with_state: bool = False):
    """Inputs of the block's causal depthwise convolution.

    x ~ N(0, 1) [batch, seqlen, d_inner] and, with ``with_state``, a cache of earlier
    inputs ~ N(0, 1) [batch, d_inner, d_conv], both rounded to ``dtype``; weight
    [d_inner, d_conv] and bias [d_inner] ~ U(-1/sqrt(d_conv), 1/sqrt(d_conv)) in fp32,
    the default initialisation range of a depthwise Conv1d (fan-in d_conv).
    """
    bound = 1.0 / np.sqrt(d_conv)
    uni = lambda g, n: g.uniform(-bound, bound, n)
    out = {
        "x": _to_dtype(_normal((batch, seqlen, d_inner), seed, _T_X), dtype),
        "weight": _fill((d_inner, d_conv), seed, _T_CW, uni),
        "bias": _fill((d_inner,), seed, _T_CB, uni),
        "dtype": dtype,
    }
    if with_state:
        out["conv_state"] = _to_dtype(_normal((batch, d_inner, d_conv), seed, _T_CS), dtype)
    return out


def initial_state(batch: int, d_inner: int, d_state: int = 16, seed: int = 0) -> np.ndarray:
    """A stored scan state [batch, d_inner, d_state] ~ N(0, 1), fp32."""
    return _normal((batch, d_inner, d_state), seed, _T_H0)


def _esize(dtype: str) -> int:
    return {"f32": 4, "bf16": 2}[dtype]


def scan_algorithmic_bytes(batch, seqlen, d_inner, d_state, in_dtype, out_dtype, with_z=True) -> int:
    """Bytes a scan must move at minimum: x, delta, (z), B, C read once and out written once."""
    si, so = _esize(in_dtype), _esize(out_dtype)
    e = batch * seqlen * d_inner
    nread = 3 if with_z else 2
    return e * (nread * si + so) + 2 * batch * seqlen * d_state * si


def decode_algorithmic_bytes(batch, d_inner, d_state, in_dtype, out_dtype, with_z=True) -> int:
    """Bytes one decode step must move: state read + written (fp32), x, delta, (z), B, C, out."""
    si, so = _esize(in_dtype), _esize(out_dtype)
    e = batch * d_inner
    nread = 3 if with_z else 2
    return e * (2 * 4 * d_state + nread * si + so) + 2 * batch * d_state * si


def conv_algorithmic_bytes(batch, seqlen, d_inner, d_conv, in_dtype, out_dtype) -> int:
    """Bytes a convolution prefill must move: x read once, out written once (the
    filter, bias and caches, a few KiB per channel group, are excluded)."""
    return batch * seqlen * d_inner * (_esize(in_dtype) + _esize(out_dtype))


def ssd_inputs(cfg: SsdConfig, seed: int = 0, batch: int | None = None, seqlen: int | None = None,
               nheads: int | None = None, ngroups: int | None = None):
    """Inputs for ``ssm_ssd_fwd`` under ``cfg`` (sizes may be overridden).

    Recipe: A[h] = -exp(U(0, log 16)) per head (decay rates 1..16, fp32); D ~ U(0.5, 1.5)
    per channel; the step drawn as for the Mamba-1 scan but per (b, t, head), with a
    per-head bias, so softplus(dt + bias) is log-uniform in [dmin, dmax]; x, z ~ N(0, 1)
    [batch, L, nheads, headdim]; B, C ~ N(0, 1) [batch, L, ngroups, d_state]; all but A,
    D and the bias rounded to the input dtype.
    """
    bsz = cfg.batch if batch is None else batch
    L = cfg.seqlen if seqlen is None else seqlen
    H = cfg.nheads if nheads is None else nheads
    G = cfg.ngroups if ngroups is None else ngroups
    P, N, dt = cfg.headdim, cfg.d_state, cfg.dtype
    A = (-np.exp(_gen(seed, _T_SA, 0).uniform(0.0, math.log(16.0), size=H))).astype(np.float32)
    D = _gen(seed, _T_SD, 0).uniform(0.5, 1.5, size=H * P).astype(np.float32)
    beta = _log_uniform64(_gen(seed, _T_BETA, 0), H, cfg.dmin, cfg.dmax)
    bias = np.log(np.expm1(beta)).astype(np.float32)
    shape = (bsz, L, H, P)
    return {
        "x": _to_dtype(_normal(shape, seed, _T_X), dt),
        "dt": _to_dtype(_delta((bsz, L, H), bias, cfg.dmin, cfg.dmax, seed, _T_DT), dt),
        "z": _to_dtype(_normal(shape, seed, _T_Z), dt),
        "B": _to_dtype(_normal((bsz, L, G, N), seed, _T_B), dt),
        "C": _to_dtype(_normal((bsz, L, G, N), seed, _T_C), dt),
        "A": A, "D": D, "dt_bias": bias, "dtype": dt,
    }


def ssd_initial_state(batch: int, nheads: int, headdim: int, d_state: int, seed: int = 0) -> np.ndarray:
    """A stored Mamba-2 state [batch, nheads, headdim, d_state] ~ N(0, 1), fp32."""
    return _normal((batch, nheads, headdim, d_state), seed, _T_H0)


def ssd_algorithmic_bytes(batch, seqlen, nheads, headdim, ngroups, d_state, in_dtype, out_dtype,
                          with_z=True) -> int:
    """Bytes a Mamba-2 scan must move at minimum: x, (z), dt, B, C read once, out written once."""
    si, so = _esize(in_dtype), _esize(out_dtype)
    e = batch * seqlen * nheads * headdim
    nread = 2 if with_z else 1
    return e * (nread * si + so) + batch * seqlen * (nheads + 2 * ngroups * d_state) * si
