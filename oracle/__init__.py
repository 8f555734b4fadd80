"""fp64 CPU oracle of the selective-SSM scan -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it, and it
shares no code with the library; both sides only share the seeded input
generator in ``workloads``.

The arithmetic lives in ``oracle.c`` (plain C, double precision); this module
only converts numpy arrays to contiguous float64 (exact for fp32 and bf16
values) and calls it through ctypes.  ``oracle.c`` names the pages each
function follows.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


class OracleLib:
    """ctypes binding of one compiled copy of ``oracle.c``."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_scan_fwd.restype = ctypes.c_int
        lib.oracle_scan_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int, _dp, _dp,
                                        _i64, _i64, _i64, _i64, _i64, ctypes.c_int]
        lib.oracle_scan_fwd_from.restype = ctypes.c_int
        lib.oracle_scan_fwd_from.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int, ctypes.c_int,
                                             _dp, _dp, _dp, _i64, _i64, _i64, _i64, _i64, ctypes.c_int]
        lib.oracle_scan_bwd.restype = ctypes.c_int
        lib.oracle_scan_bwd.argtypes = [_dp] * 8 + [ctypes.c_int] + [_dp] * 12 + [_i64] * 4
        lib.oracle_conv1d_fwd.restype = ctypes.c_int
        lib.oracle_conv1d_fwd.argtypes = [_dp, _dp, _dp, ctypes.c_int, _dp, _dp, _dp, _i64, _i64, _i64, _i64]
        lib.oracle_conv1d_update.restype = ctypes.c_int
        lib.oracle_conv1d_update.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_int, _dp, _i64, _i64, _i64]
        lib.oracle_state_update.restype = ctypes.c_int
        lib.oracle_state_update.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int,
                                            ctypes.c_int, _dp, _i64, _i64, _i64]
        lib.oracle_affine_compose.restype = None
        lib.oracle_affine_compose.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _i64]
        lib.oracle_step_size.restype = None
        lib.oracle_step_size.argtypes = [_dp, _dp, ctypes.c_int, _dp, _i64, _i64]
        lib.oracle_ssd_fwd.restype = ctypes.c_int
        lib.oracle_ssd_fwd.argtypes = [_dp] * 8 + [ctypes.c_int] + [_dp] * 3 + [_i64] * 6 + [ctypes.c_int]
        lib.oracle_ssd_state_update.restype = ctypes.c_int
        lib.oracle_ssd_state_update.argtypes = [_dp] * 9 + [ctypes.c_int, _dp] + [_i64] * 5
        lib.oracle_abi_version.restype = ctypes.c_int
        self.path = path
        self.lib = lib

    def scan_fwd(self, x, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True,
                 chunk: int = 0, nthreads: int | None = None, return_state: bool = True, h0=None,
                 zoh: bool = False):
        """Sequential fp64 scan from the state h0 [batch, d_inner, d_state] (None: zero).

        x, delta, z: [batch, L, d_inner]; B, C: [batch, L, d_state]; A: [d_inner, d_state];
        D, delta_bias: [d_inner].  Returns (out [batch, L, d_inner], last_state
        [batch, d_inner, d_state] or None), float64.  ``chunk > 0`` runs the chunked
        form: per-chunk affine pairs composed in time order, then each chunk re-run.
        ``zoh`` uses the exact zero-order-hold input coefficient (e^{dt A} - 1) / A
        in place of dt."""
        x, delta, A, B, C = map(_f64, (x, delta, A, B, C))
        D, z, delta_bias, h0 = map(_f64, (D, z, delta_bias, h0))
        if x.ndim != 3:
            raise ValueError("x must be [batch, L, d_inner]")
        batch, L, Dn = x.shape
        N = A.shape[1]
        if delta.shape != x.shape or (z is not None and z.shape != x.shape):
            raise ValueError("delta and z must match x")
        if A.shape != (Dn, N) or B.shape != (batch, L, N) or C.shape != (batch, L, N):
            raise ValueError("bad A/B/C shape")
        if (D is not None and D.shape != (Dn,)) or (delta_bias is not None and delta_bias.shape != (Dn,)):
            raise ValueError("bad D/delta_bias shape")
        if h0 is not None and h0.shape != (batch, Dn, N):
            raise ValueError("h0 must be [batch, d_inner, d_state]")
        out = np.empty((batch, L, Dn), dtype=np.float64)
        last = np.empty((batch, Dn, N), dtype=np.float64) if return_state else None
        rc = self.lib.oracle_scan_fwd_from(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                           _ptr(delta_bias), int(bool(softplus)), int(bool(zoh)), _ptr(h0),
                                           _ptr(out), _ptr(last),
                                           batch, L, Dn, N, int(chunk), int(nthreads or default_threads()))
        if rc != 0:
            raise ValueError("oracle_scan_fwd rejected its arguments")
        return out, last

    def state_update(self, state, x, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True,
                     zoh: bool = False):
        """One decode step.  state: [batch, d_inner, d_state]; x, delta, z: [batch, d_inner];
        B, C: [batch, d_state].  Returns (out [batch, d_inner], new_state) as float64; the
        ``state`` argument itself is not modified."""
        st = np.array(state, dtype=np.float64, order="C", copy=True)
        x, delta, A, B, C = map(_f64, (x, delta, A, B, C))
        D, z, delta_bias = map(_f64, (D, z, delta_bias))
        batch, Dn = x.shape
        N = A.shape[1]
        if st.shape != (batch, Dn, N) or B.shape != (batch, N) or C.shape != (batch, N):
            raise ValueError("bad state/B/C shape")
        out = np.empty((batch, Dn), dtype=np.float64)
        rc = self.lib.oracle_state_update(_ptr(st), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                          _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(softplus)),
                                          int(bool(zoh)), _ptr(out), batch, Dn, N)
        if rc != 0:
            raise ValueError("oracle_state_update rejected its arguments")
        return out, st

    def ssd_fwd(self, x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus=True, h0=None,
                nthreads: int | None = None, return_state: bool = True):
        """Mamba-2 (SSD) scan, sequential fp64, from h0 [batch, nheads, headdim, d_state]
        (None: zero).  x, z: [batch, L, nheads, headdim]; dt: [batch, L, nheads]; B, C:
        [batch, L, ngroups, d_state]; A, dt_bias: [nheads]; D: [nheads * headdim].
        Returns (out [batch, L, nheads, headdim], last_state or None), float64."""
        x, dt, A, B, C = map(_f64, (x, dt, A, B, C))
        D, z, dt_bias, h0 = map(_f64, (D, z, dt_bias, h0))
        if x.ndim != 4 or B.ndim != 4:
            raise ValueError("x must be [batch, L, nheads, headdim] and B [batch, L, ngroups, d_state]")
        batch, L, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        if dt.shape != (batch, L, H) or A.shape != (H,) or B.shape != (batch, L, G, N) or C.shape != B.shape:
            raise ValueError("bad dt/A/B/C shape")
        if (z is not None and z.shape != x.shape) or (D is not None and D.shape != (H * P,)):
            raise ValueError("bad z/D shape")
        if (dt_bias is not None and dt_bias.shape != (H,)) or (h0 is not None and h0.shape != (batch, H, P, N)):
            raise ValueError("bad dt_bias/h0 shape")
        out = np.empty(x.shape, dtype=np.float64)
        last = np.empty((batch, H, P, N), dtype=np.float64) if return_state else None
        rc = self.lib.oracle_ssd_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
                                     int(bool(softplus)), _ptr(h0), _ptr(out), _ptr(last), batch, L, H, P, G, N,
                                     int(nthreads or default_threads()))
        if rc != 0:
            raise ValueError("oracle_ssd_fwd rejected its arguments")
        return out, last

    def ssd_state_update(self, state, x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus=True):
        """One Mamba-2 decode step.  state: [batch, nheads, headdim, d_state]; x, z:
        [batch, nheads, headdim]; dt: [batch, nheads]; B, C: [batch, ngroups, d_state].
        Returns (out, new_state) as float64; ``state`` itself is not modified."""
        st = np.array(state, dtype=np.float64, order="C", copy=True)
        x, dt, A, B, C = map(_f64, (x, dt, A, B, C))
        D, z, dt_bias = map(_f64, (D, z, dt_bias))
        batch, H, P = x.shape
        G, N = B.shape[1], B.shape[2]
        if st.shape != (batch, H, P, N) or dt.shape != (batch, H) or C.shape != B.shape:
            raise ValueError("bad state/dt/B/C shape")
        out = np.empty(x.shape, dtype=np.float64)
        rc = self.lib.oracle_ssd_state_update(_ptr(st), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                              _ptr(z), _ptr(dt_bias), int(bool(softplus)), _ptr(out), batch, H, P,
                                              G, N)
        if rc != 0:
            raise ValueError("oracle_ssd_state_update rejected its arguments")
        return out, st

    def affine_compose(self, later, earlier):
        """(a2, b2) o (a1, b1) = (a2*a1, a2*b1 + b2): ``earlier`` acts first, then ``later``."""
        a2, b2 = (np.atleast_1d(_f64(v)) for v in later)
        a1, b1 = (np.atleast_1d(_f64(v)) for v in earlier)
        n = a2.size
        a = np.empty(n)
        b = np.empty(n)
        self.lib.oracle_affine_compose(_ptr(a2), _ptr(b2), _ptr(a1), _ptr(b1), _ptr(a), _ptr(b), n)
        return a, b

    def scan_bwd(self, x, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, h0=None,
                 dout=None, dlast=None):
        """Gradients of the scan for the output gradient dout [batch, L, d_inner] (and
        optionally dlast [batch, d_inner, d_state], the gradient of the final state).
        Returns a dict of float64 arrays: dx, ddelta, dA, dB, dC, and dD, dz,
        ddelta_bias, dh0 for the optional inputs that were given."""
        x, delta, A, B, C = map(_f64, (x, delta, A, B, C))
        D, z, delta_bias, h0, dout, dlast = map(_f64, (D, z, delta_bias, h0, dout, dlast))
        batch, L, Dn = x.shape
        N = A.shape[1]
        if dout is None or dout.shape != x.shape:
            raise ValueError("dout must match x")
        g = {k: np.empty(x.shape) for k in ("dx", "ddelta")}
        g["dA"] = np.empty((Dn, N))
        g["dB"] = np.empty((batch, L, N))
        g["dC"] = np.empty((batch, L, N))
        g["dD"] = np.empty(Dn) if D is not None else None
        g["dz"] = np.empty(x.shape) if z is not None else None
        g["ddelta_bias"] = np.empty(Dn) if delta_bias is not None else None
        g["dh0"] = np.empty((batch, Dn, N)) if h0 is not None else None
        rc = self.lib.oracle_scan_bwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                      _ptr(delta_bias), int(bool(softplus)), _ptr(h0), _ptr(dout), _ptr(dlast),
                                      _ptr(g["dx"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
                                      _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["ddelta_bias"]), _ptr(g["dh0"]),
                                      batch, L, Dn, N)
        if rc != 0:
            raise ValueError("oracle_scan_bwd rejected its arguments")
        return {k: v for k, v in g.items() if v is not None}

    def conv1d_fwd(self, x, weight, bias=None, silu=True, conv_state=None, return_state=True):
        """Causal depthwise conv1d (+ bias, + SiLU).  x: [batch, L, d_inner]; weight:
        [d_inner, d_conv]; bias: [d_inner]; conv_state: [batch, d_inner, d_conv], the
        d_conv most recent earlier inputs, oldest first (None: zeros).  Returns (out
        [batch, L, d_inner], new conv_state or None) as float64."""
        x, w, bias, st = map(_f64, (x, weight, bias, conv_state))
        batch, L, Dn = x.shape
        K = w.shape[1]
        if w.shape != (Dn, K) or (bias is not None and bias.shape != (Dn,)):
            raise ValueError("bad weight/bias shape")
        if st is not None and st.shape != (batch, Dn, K):
            raise ValueError("conv_state must be [batch, d_inner, d_conv]")
        out = np.empty((batch, L, Dn), dtype=np.float64)
        st_out = np.empty((batch, Dn, K), dtype=np.float64) if return_state else None
        rc = self.lib.oracle_conv1d_fwd(_ptr(x), _ptr(w), _ptr(bias), int(bool(silu)), _ptr(st), _ptr(out),
                                        _ptr(st_out), batch, L, Dn, K)
        if rc != 0:
            raise ValueError("oracle_conv1d_fwd rejected its arguments")
        return out, st_out

    def conv1d_update(self, conv_state, x, weight, bias=None, silu=True):
        """One decode step of the convolution.  conv_state: [batch, d_inner, d_conv];
        x: [batch, d_inner].  Returns (out [batch, d_inner], new conv_state); the
        argument itself is not modified."""
        st = np.array(conv_state, dtype=np.float64, order="C", copy=True)
        x, w, bias = map(_f64, (x, weight, bias))
        batch, Dn = x.shape
        K = w.shape[1]
        if st.shape != (batch, Dn, K) or w.shape != (Dn, K):
            raise ValueError("bad conv_state/weight shape")
        out = np.empty((batch, Dn), dtype=np.float64)
        rc = self.lib.oracle_conv1d_update(_ptr(st), _ptr(x), _ptr(w), _ptr(bias), int(bool(silu)), _ptr(out),
                                           batch, Dn, K)
        if rc != 0:
            raise ValueError("oracle_conv1d_update rejected its arguments")
        return out, st

    def step_size(self, delta, delta_bias=None, softplus=True):
        """dt = softplus(delta + bias), or delta + bias; delta: [rows, d_inner]."""
        d = _f64(np.atleast_2d(delta))
        bias = _f64(delta_bias)
        out = np.empty_like(d)
        self.lib.oracle_step_size(_ptr(d), _ptr(bias), int(bool(softplus)), _ptr(out), d.shape[0], d.shape[1])
        return out


_default: OracleLib | None = None


def load() -> OracleLib:
    """The oracle built from ``oracle.c`` (compiled first if missing or stale)."""
    global _default
    if _default is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        _default = OracleLib(path)
    return _default


def scan_fwd(*args, **kw):
    return load().scan_fwd(*args, **kw)


def state_update(*args, **kw):
    return load().state_update(*args, **kw)


def affine_compose(*args, **kw):
    return load().affine_compose(*args, **kw)


def step_size(*args, **kw):
    return load().step_size(*args, **kw)


def conv1d_fwd(*args, **kw):
    return load().conv1d_fwd(*args, **kw)


def conv1d_update(*args, **kw):
    return load().conv1d_update(*args, **kw)


def scan_bwd(*args, **kw):
    return load().scan_bwd(*args, **kw)


def ssd_fwd(*args, **kw):
    return load().ssd_fwd(*args, **kw)


def ssd_state_update(*args, **kw):
    return load().ssd_state_update(*args, **kw)
