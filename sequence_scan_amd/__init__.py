"""Python binding of libssmscan (the selective-SSM scan on MI355X).

Argument marshalling only: tensors are passed to the C ABI as device
pointers, sizes and the current HIP stream; every step of the computation
runs in the library's gfx950 kernels.  PyTorch provides device memory and
streams.  There is no fallback: if ``libssmscan.so`` is missing or cannot be
loaded, every call raises.

Functions carry the C names: ``ssm_scan_fwd``, ``ssm_state_update``,
``ssm_scan_fwd_plan``, ``ssm_scan_fwd_from``, ``ssm_scan_plan``,
``ssm_scan_bwd``, ``ssm_scan_bwd_plan``, ``ssm_scan_bwd_plan_query``, ``ssm_conv1d_fwd``,
``ssm_conv1d_update``, ``ssm_ssd_fwd``, ``ssm_ssd_fwd_plan``, ``ssm_ssd_plan_query``, ``ssm_ssd_state_update``,
``ssm_affine_exclusive_scan``,
``ssm_scan_ckpt_bytes``, ``ssm_scan_fwd_ckpt``, ``ssm_scan_bwd_ckpt`` (``ssm_scan_bwd(..., ckpt=)``),
``ssm_status_string``, ``ssm_last_error``, ``ssm_abi_version``, ``ssm_trim_workspace``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssmscan.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "ssmscan.h")

SSM_F32 = 0
SSM_BF16 = 1
SSM_SOFTPLUS = 1  # step flags: dt = softplus(delta + bias)
SSM_ZOH = 2       # step flags: exact zero-order-hold input coefficient
SSM_OK, SSM_ERR_NULL_ARG, SSM_ERR_BAD_SHAPE, SSM_ERR_UNSUPPORTED, SSM_ERR_HIP = range(5)
STATUS_NAMES = {0: "SSM_OK", 1: "SSM_ERR_NULL_ARG", 2: "SSM_ERR_BAD_SHAPE", 3: "SSM_ERR_UNSUPPORTED",
                4: "SSM_ERR_HIP"}
D_STATE = 16


class SSMError(RuntimeError):
    """A non-OK status from libssmscan; ``status`` holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class ssm_plan(ctypes.Structure):
    _fields_ = [("states_per_wave", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("chunk_len", ctypes.c_int64), ("n_chunks", ctypes.c_int64),
                ("reserved", ctypes.c_int64 * 4)]


_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libssmscan.so is not built ({LIB_PATH}); run sequence_scan_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    scan_args = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp,
                 _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp]
    lib.ssm_scan_fwd.argtypes = scan_args
    lib.ssm_scan_fwd.restype = ctypes.c_int
    lib.ssm_scan_fwd_plan.argtypes = scan_args + [ctypes.POINTER(ssm_plan)]
    lib.ssm_scan_fwd_plan.restype = ctypes.c_int
    lib.ssm_scan_fwd_from.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
                                      _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp,
                                      ctypes.POINTER(ssm_plan)]
    lib.ssm_scan_fwd_from.restype = ctypes.c_int
    lib.ssm_scan_fwd_noalloc.argtypes = lib.ssm_scan_fwd_from.argtypes
    lib.ssm_scan_fwd_noalloc.restype = ctypes.c_int
    lib.ssm_scan_bwd.argtypes = [_vp] * 8 + [ctypes.c_int] + [_vp] * 12 + [_i64] * 4 + [ctypes.c_int, ctypes.c_int, _vp]
    lib.ssm_scan_bwd.restype = ctypes.c_int
    lib.ssm_scan_bwd_plan.argtypes = lib.ssm_scan_bwd.argtypes + [ctypes.POINTER(ssm_plan)]
    lib.ssm_scan_bwd_plan.restype = ctypes.c_int
    lib.ssm_scan_ckpt_bytes.argtypes = [_i64, _i64, _i64, _i64, ctypes.POINTER(ctypes.c_int64)]
    lib.ssm_scan_ckpt_bytes.restype = ctypes.c_int
    lib.ssm_scan_fwd_ckpt.argtypes = [_vp] * 8 + [ctypes.c_int] + [_vp] * 4 + [_i64] * 4 + [ctypes.c_int,
                                                                                       ctypes.c_int, _vp]
    lib.ssm_scan_fwd_ckpt.restype = ctypes.c_int
    lib.ssm_scan_bwd_ckpt.argtypes = [_vp] * 8 + [ctypes.c_int] + [_vp] * 13 + [_i64] * 4 + [ctypes.c_int,
                                                                                        ctypes.c_int, _vp]
    lib.ssm_scan_bwd_ckpt.restype = ctypes.c_int
    lib.ssm_scan_bwd_plan_query.argtypes = [_i64, _i64, _i64, _i64, ctypes.POINTER(ssm_plan)]
    lib.ssm_scan_bwd_plan_query.restype = ctypes.c_int
    lib.ssm_conv1d_fwd.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                   ctypes.c_int, ctypes.c_int, _vp]
    lib.ssm_conv1d_fwd.restype = ctypes.c_int
    lib.ssm_conv1d_update.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int, _vp, _i64, _i64, _i64,
                                      ctypes.c_int, ctypes.c_int, _vp]
    lib.ssm_conv1d_update.restype = ctypes.c_int
    lib.ssm_state_update.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp,
                                     _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp]
    lib.ssm_state_update.restype = ctypes.c_int
    lib.ssm_ssd_fwd.argtypes = [_vp] * 8 + [ctypes.c_int, _vp, _vp, _vp] + [_i64] * 6 + [ctypes.c_int, ctypes.c_int,
                                                                                         _vp]
    lib.ssm_ssd_fwd.restype = ctypes.c_int
    lib.ssm_ssd_fwd_plan.argtypes = lib.ssm_ssd_fwd.argtypes + [ctypes.POINTER(ssm_plan)]
    lib.ssm_ssd_fwd_plan.restype = ctypes.c_int
    lib.ssm_ssd_plan_query.argtypes = [_i64] * 6 + [ctypes.POINTER(ssm_plan)]
    lib.ssm_ssd_plan_query.restype = ctypes.c_int
    lib.ssm_ssd_state_update.argtypes = [_vp] * 9 + [ctypes.c_int, _vp] + [_i64] * 5 + [ctypes.c_int, ctypes.c_int,
                                                                                      _vp]
    lib.ssm_ssd_state_update.restype = ctypes.c_int
    lib.ssm_scan_plan.argtypes = [_i64, _i64, _i64, _i64, ctypes.POINTER(ssm_plan)]
    lib.ssm_scan_plan.restype = ctypes.c_int
    lib.ssm_affine_exclusive_scan.argtypes = [_vp, _vp, _vp, _vp, _i64, _vp]
    lib.ssm_affine_exclusive_scan.restype = ctypes.c_int
    lib.ssm_status_string.argtypes = [ctypes.c_int]
    lib.ssm_status_string.restype = ctypes.c_char_p
    lib.ssm_last_error.argtypes = []
    lib.ssm_last_error.restype = ctypes.c_char_p
    lib.ssm_abi_version.argtypes = []
    lib.ssm_abi_version.restype = ctypes.c_int
    lib.ssm_trim_workspace.argtypes = []
    lib.ssm_trim_workspace.restype = ctypes.c_int
    _lib = lib
    return lib


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


def _check(status: int):
    if status != SSM_OK:
        raise SSMError(status, _load().ssm_last_error().decode())


def _flags(softplus, zoh) -> int:
    """The step-flags word of the C ABI."""
    return (SSM_SOFTPLUS if softplus else 0) | (SSM_ZOH if zoh else 0)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return SSM_F32
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _expect(like, **tensors):
    """Check each named tensor against (shape, dtype) before its pointer reaches the
    C ABI, which trusts the sizes it is given: a mismatch would make the kernels read
    or write past a tensor.  dtype None accepts float32 or bfloat16; every tensor
    must be on ``like``'s device.  None tensors (optional inputs) are skipped."""
    import torch
    for name, spec in tensors.items():
        t, shape, dtype = spec
        if t is None:
            continue
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if dtype is None:
            if t.dtype not in (torch.float32, torch.bfloat16):
                raise TypeError(f"{name} must be float32 or bfloat16, got {t.dtype}")
        elif t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if t.device != like.device:
            raise ValueError(f"{name} is on {t.device}, expected {like.device}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def ssm_status_string(status: int) -> str:
    return _load().ssm_status_string(int(status)).decode()


def ssm_last_error() -> str:
    return _load().ssm_last_error().decode()


def ssm_abi_version() -> int:
    return int(_load().ssm_abi_version())


def ssm_trim_workspace() -> None:
    """Return the workspace memory the library's pool on the current device holds
    unused to the system (call after synchronising)."""
    _check(_load().ssm_trim_workspace())


def ssm_scan_plan(batch: int, seqlen: int, d_inner: int, d_state: int = D_STATE) -> dict:
    """The plan ``ssm_scan_fwd`` picks for these sizes."""
    p = ssm_plan()
    _check(_load().ssm_scan_plan(batch, seqlen, d_inner, d_state, ctypes.byref(p)))
    return {"states_per_wave": p.states_per_wave, "chunk_len": p.chunk_len, "n_chunks": p.n_chunks}


def ssm_scan_fwd(x, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True,
                 out=None, last_state=None, out_dtype=None, stream=None, plan: Optional[dict] = None,
                 zoh: bool = False):
    """Forward selective scan from a zero state (see include/ssmscan.h).

    x, delta, z: [batch, seqlen, d_inner]; B, C: [batch, seqlen, d_state] (all float32 or
    all bfloat16); A: [d_inner, d_state], D, delta_bias: [d_inner] (float32).  ``out``
    (allocated if None, dtype ``out_dtype`` or x's) and ``last_state`` (float32
    [batch, d_inner, d_state], optional) are written on the current stream.  ``plan`` =
    {"states_per_wave": .., "chunk_len": ..} forces an execution plan.  ``zoh`` selects the
    exact zero-order-hold input coefficient (e^{dt A} - 1) / A in place of dt.  Returns out.
    """
    import torch
    if x.dim() != 3:
        raise ValueError("x must be [batch, seqlen, d_inner]")
    batch, seqlen, d_inner = x.shape
    if A.dim() != 2:
        raise ValueError("A must be [d_inner, d_state]")
    d_state = A.shape[1]
    f32, xs, bcs, st = torch.float32, (batch, seqlen, d_inner), (batch, seqlen, d_state), (batch, d_inner, d_state)
    _expect(x, x=(x, xs, None), delta=(delta, xs, x.dtype), z=(z, xs, x.dtype), B=(B, bcs, x.dtype),
            C=(C, bcs, x.dtype), A=(A, (d_inner, d_state), f32), D=(D, (d_inner,), f32),
            delta_bias=(delta_bias, (d_inner,), f32), out=(out, xs, None), last_state=(last_state, st, f32))
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    lib = _load()
    args = (_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            _flags(softplus, zoh), _ptr(out), _ptr(last_state), batch, seqlen, d_inner, d_state,
            _dtype_code(x), _dtype_code(out), _stream(stream))
    if plan is None:
        _check(lib.ssm_scan_fwd(*args))
    else:
        p = ssm_plan()
        p.states_per_wave = int(plan["states_per_wave"])
        p.chunk_len = int(plan["chunk_len"])
        _check(lib.ssm_scan_fwd_plan(*args, ctypes.byref(p)))
    return out


def ssm_scan_fwd_plan(*args, plan: dict, **kw):
    return ssm_scan_fwd(*args, plan=plan, **kw)


def _plan_struct(plan: Optional[dict]):
    if plan is None:
        return None
    p = ssm_plan()
    p.states_per_wave = int(plan["states_per_wave"])
    p.chunk_len = int(plan["chunk_len"])
    return ctypes.byref(p)


def ssm_scan_fwd_from(x, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True,
                      initial_state=None, out=None, last_state=None, out_dtype=None, stream=None,
                      plan: Optional[dict] = None, zoh: bool = False):
    """Forward scan continuing from ``initial_state`` [batch, d_inner, d_state] float32
    (None: zero); ``last_state`` may be the same tensor (replaced in place).  Other
    arguments as for ``ssm_scan_fwd``.  Returns out."""
    return _scan_from("ssm_scan_fwd_from", x, delta, A, B, C, D, z, delta_bias, softplus, initial_state, out,
                      last_state, out_dtype, stream, plan, zoh)


def ssm_scan_ckpt_bytes(batch: int, seqlen: int, d_inner: int, d_state: int = D_STATE) -> int:
    """Bytes of the backward's checkpoints for these sizes (``ssm_scan_fwd_ckpt``)."""
    n = ctypes.c_int64(0)
    _check(_load().ssm_scan_ckpt_bytes(batch, seqlen, d_inner, d_state, ctypes.byref(n)))
    return int(n.value)


def ssm_scan_fwd_ckpt(x, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True,
                      initial_state=None, out=None, last_state=None, ckpt=None, out_dtype=None, stream=None):
    """``ssm_scan_fwd_from`` that also keeps the backward's checkpoints.  Returns
    (out, ckpt); ``ckpt`` (a uint8 device tensor of ``ssm_scan_ckpt_bytes`` bytes) is
    allocated if None.  Pass it to ``ssm_scan_bwd(..., ckpt=ckpt)`` with the same inputs."""
    import torch
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be [batch, seqlen, d_inner] and A [d_inner, d_state]")
    batch, seqlen, d_inner = x.shape
    d_state = A.shape[1]
    f32, xs, bcs, st = torch.float32, (batch, seqlen, d_inner), (batch, seqlen, d_state), (batch, d_inner, d_state)
    _expect(x, x=(x, xs, None), delta=(delta, xs, x.dtype), z=(z, xs, x.dtype), B=(B, bcs, x.dtype),
            C=(C, bcs, x.dtype), A=(A, (d_inner, d_state), f32), D=(D, (d_inner,), f32),
            delta_bias=(delta_bias, (d_inner,), f32), out=(out, xs, None), last_state=(last_state, st, f32),
            initial_state=(initial_state, st, f32))
    nbytes = ssm_scan_ckpt_bytes(batch, seqlen, d_inner, d_state)
    if ckpt is None:
        ckpt = torch.empty((nbytes,), dtype=torch.uint8, device=x.device)
    elif ckpt.numel() * ckpt.element_size() < nbytes or not ckpt.is_contiguous() or ckpt.device != x.device:
        raise ValueError(f"ckpt must be a contiguous tensor of at least {nbytes} bytes on {x.device}")
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    _check(_load().ssm_scan_fwd_ckpt(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                     _ptr(delta_bias), int(bool(softplus)), _ptr(initial_state), _ptr(out),
                                     _ptr(last_state), _ptr(ckpt), batch, seqlen, d_inner, d_state,
                                     _dtype_code(x), _dtype_code(out), _stream(stream)))
    return out, ckpt


def ssm_scan_fwd_noalloc(x, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True,
                         initial_state=None, out=None, last_state=None, out_dtype=None, stream=None,
                         plan: Optional[dict] = None, zoh: bool = False):
    """``ssm_scan_fwd_from`` whose carry workspace is the library's fixed per-device
    scratch (SSM_NOALLOC_SCRATCH_BYTES) instead of a stream-ordered allocation.  The C
    call allocates nothing; pass ``out`` to keep this wrapper from allocating it."""
    return _scan_from("ssm_scan_fwd_noalloc", x, delta, A, B, C, D, z, delta_bias, softplus, initial_state, out,
                      last_state, out_dtype, stream, plan, zoh)


def _scan_from(fn, x, delta, A, B, C, D, z, delta_bias, softplus, initial_state, out, last_state, out_dtype,
               stream, plan, zoh):
    import torch
    if x.dim() != 3:
        raise ValueError("x must be [batch, seqlen, d_inner]")
    batch, seqlen, d_inner = x.shape
    if A.dim() != 2:
        raise ValueError("A must be [d_inner, d_state]")
    d_state = A.shape[1]
    f32, xs, bcs, st = torch.float32, (batch, seqlen, d_inner), (batch, seqlen, d_state), (batch, d_inner, d_state)
    _expect(x, x=(x, xs, None), delta=(delta, xs, x.dtype), z=(z, xs, x.dtype), B=(B, bcs, x.dtype),
            C=(C, bcs, x.dtype), A=(A, (d_inner, d_state), f32), D=(D, (d_inner,), f32),
            delta_bias=(delta_bias, (d_inner,), f32), out=(out, xs, None), last_state=(last_state, st, f32),
            initial_state=(initial_state, st, f32))
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    _check(getattr(_load(), fn)(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                _ptr(delta_bias), _flags(softplus, zoh), _ptr(initial_state), _ptr(out),
                                _ptr(last_state), batch, seqlen, d_inner, d_state, _dtype_code(x),
                                _dtype_code(out), _stream(stream), _plan_struct(plan)))
    return out


def ssm_scan_bwd_plan(*args, plan: dict, **kw):
    return ssm_scan_bwd(*args, plan=plan, **kw)


def ssm_scan_bwd_plan_query(batch: int, seqlen: int, d_inner: int, d_state: int = D_STATE) -> dict:
    """The plan ``ssm_scan_bwd`` picks for these sizes (its time chunks)."""
    p = ssm_plan()
    _check(_load().ssm_scan_bwd_plan_query(batch, seqlen, d_inner, d_state, ctypes.byref(p)))
    return {"states_per_wave": p.states_per_wave, "chunk_len": p.chunk_len, "n_chunks": p.n_chunks}


def ssm_scan_bwd(x, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True, initial_state=None,
                 dout=None, dlast_state=None, want_dinitial_state: bool = False, grad_dtype=None, stream=None,
                 plan: Optional[dict] = None, ckpt=None):
    """Gradients of the scan (see include/ssmscan.h).  Forward inputs as for
    ``ssm_scan_fwd_from``; ``dout`` [batch, seqlen, d_inner] (its dtype is the gradient
    dtype unless ``grad_dtype`` is given); ``dlast_state`` optional.  Returns a dict with
    dx, ddelta, dA, dB, dC and, for the inputs given, dD, dz, ddelta_bias, and
    dinitial_state when ``want_dinitial_state``.  ``plan`` = {"states_per_wave": 4,
    "chunk_len": ..} forces the time chunks (``ssm_scan_bwd_plan``).  ``ckpt``: the
    checkpoints of ``ssm_scan_fwd_ckpt`` over the same inputs (``ssm_scan_bwd_ckpt``:
    the forward is not run again)."""
    import torch
    if x.dim() != 3 or dout is None:
        raise ValueError("x must be [batch, seqlen, d_inner] and dout given")
    batch, seqlen, d_inner = x.shape
    if A.dim() != 2:
        raise ValueError("A must be [d_inner, d_state]")
    d_state = A.shape[1]
    gdt = grad_dtype or dout.dtype
    if dout.dtype != gdt:
        raise TypeError("dout must have the gradient dtype")
    f32, xs, bcs, st = torch.float32, (batch, seqlen, d_inner), (batch, seqlen, d_state), (batch, d_inner, d_state)
    _expect(x, x=(x, xs, None), delta=(delta, xs, x.dtype), z=(z, xs, x.dtype), B=(B, bcs, x.dtype),
            C=(C, bcs, x.dtype), A=(A, (d_inner, d_state), f32), D=(D, (d_inner,), f32),
            delta_bias=(delta_bias, (d_inner,), f32), initial_state=(initial_state, st, f32),
            dout=(dout, xs, None), dlast_state=(dlast_state, st, f32))
    dev = x.device
    g = {"dx": torch.empty(x.shape, dtype=gdt, device=dev), "ddelta": torch.empty(x.shape, dtype=gdt, device=dev),
         "dA": torch.empty(A.shape, dtype=torch.float32, device=dev),
         "dB": torch.empty(B.shape, dtype=gdt, device=dev), "dC": torch.empty(C.shape, dtype=gdt, device=dev)}
    if D is not None:
        g["dD"] = torch.empty(D.shape, dtype=torch.float32, device=dev)
    if z is not None:
        g["dz"] = torch.empty(x.shape, dtype=gdt, device=dev)
    if delta_bias is not None:
        g["ddelta_bias"] = torch.empty(delta_bias.shape, dtype=torch.float32, device=dev)
    if want_dinitial_state:
        g["dinitial_state"] = torch.empty((batch, d_inner, d_state), dtype=torch.float32, device=dev)
    args = (_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            int(bool(softplus)), _ptr(initial_state), _ptr(dout), _ptr(dlast_state), _ptr(g["dx"]),
            _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g.get("dD")), _ptr(g.get("dz")),
            _ptr(g.get("ddelta_bias")), _ptr(g.get("dinitial_state")), batch, seqlen, d_inner, d_state,
            _dtype_code(x), _dtype_code(g["dx"]), _stream(stream))
    lib = _load()
    if ckpt is not None:
        if plan is not None:
            raise ValueError("ssm_scan_bwd_ckpt runs the default plan")
        nbytes = ssm_scan_ckpt_bytes(batch, seqlen, d_inner, d_state)
        if ckpt.numel() * ckpt.element_size() < nbytes or not ckpt.is_contiguous() or ckpt.device != x.device:
            raise ValueError(f"ckpt must be a contiguous tensor of at least {nbytes} bytes on {x.device}")
        _check(lib.ssm_scan_bwd_ckpt(*args[:12], _ptr(ckpt), *args[12:]))
    elif plan is None:
        _check(lib.ssm_scan_bwd(*args))
    else:
        _check(lib.ssm_scan_bwd_plan(*args, _plan_struct(plan)))
    return g


def ssm_conv1d_fwd(x, weight, bias=None, silu: bool = True, conv_state_in=None, out=None,
                   conv_state_out=None, out_dtype=None, stream=None):
    """Causal depthwise conv1d (+ bias, + SiLU) over x [batch, seqlen, d_inner]; weight
    [d_inner, d_conv] and bias [d_inner] float32; the caches [batch, d_inner, d_conv]
    have x's dtype.  Returns out (allocated if None, dtype ``out_dtype`` or x's)."""
    import torch
    if x.dim() != 3 or weight.dim() != 2:
        raise ValueError("x must be [batch, seqlen, d_inner] and weight [d_inner, d_conv]")
    batch, seqlen, d_inner = x.shape
    K = weight.shape[1]
    f32, xs, cs = torch.float32, (batch, seqlen, d_inner), (batch, d_inner, K)
    _expect(x, x=(x, xs, None), weight=(weight, (d_inner, K), f32), bias=(bias, (d_inner,), f32),
            conv_state_in=(conv_state_in, cs, x.dtype), conv_state_out=(conv_state_out, cs, x.dtype),
            out=(out, xs, None))
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    _check(_load().ssm_conv1d_fwd(_ptr(x), _ptr(weight), _ptr(bias), int(bool(silu)), _ptr(conv_state_in),
                                  _ptr(out), _ptr(conv_state_out), batch, seqlen, d_inner, weight.shape[1],
                                  _dtype_code(x), _dtype_code(out), _stream(stream)))
    return out


def ssm_conv1d_update(conv_state, x, weight, bias=None, silu: bool = True, out=None, out_dtype=None,
                      stream=None):
    """One decode step of the convolution; ``conv_state`` [batch, d_inner, d_conv] (x's
    dtype) is updated in place.  x: [batch, d_inner].  Returns out."""
    import torch
    if x.dim() != 2 or weight.dim() != 2:
        raise ValueError("x must be [batch, d_inner] and weight [d_inner, d_conv]")
    batch, d_inner = x.shape
    K = weight.shape[1]
    _expect(x, x=(x, (batch, d_inner), None), conv_state=(conv_state, (batch, d_inner, K), x.dtype),
            weight=(weight, (d_inner, K), torch.float32), bias=(bias, (d_inner,), torch.float32),
            out=(out, (batch, d_inner), None))
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    _check(_load().ssm_conv1d_update(_ptr(conv_state), _ptr(x), _ptr(weight), _ptr(bias), int(bool(silu)),
                                     _ptr(out), batch, d_inner, weight.shape[1], _dtype_code(x), _dtype_code(out),
                                     _stream(stream)))
    return out


def ssm_state_update(state, x, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True,
                     out=None, out_dtype=None, stream=None, zoh: bool = False):
    """One decode step (see include/ssmscan.h); ``state`` [batch, d_inner, d_state] float32
    is updated in place.  x, delta, z: [batch, d_inner]; B, C: [batch, d_state]."""
    import torch
    if x.dim() != 2:
        raise ValueError("x must be [batch, d_inner]")
    batch, d_inner = x.shape
    if state.dim() != 3:
        raise ValueError("state must be [batch, d_inner, d_state]")
    d_state = state.shape[2]
    f32, xs, bcs = torch.float32, (batch, d_inner), (batch, d_state)
    _expect(x, state=(state, (batch, d_inner, d_state), f32), x=(x, xs, None), delta=(delta, xs, x.dtype),
            z=(z, xs, x.dtype), B=(B, bcs, x.dtype), C=(C, bcs, x.dtype), A=(A, (d_inner, d_state), f32),
            D=(D, (d_inner,), f32), delta_bias=(delta_bias, (d_inner,), f32), out=(out, xs, None))
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    _check(_load().ssm_state_update(_ptr(state), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                    _ptr(z), _ptr(delta_bias), _flags(softplus, zoh), _ptr(out), batch, d_inner,
                                    d_state, _dtype_code(x), _dtype_code(out), _stream(stream)))
    return out


def ssm_affine_exclusive_scan(a, b, out_a=None, out_b=None, stream=None):
    """Exclusive scan of affine pairs (a[k], b[k]) in time order on the GPU (float32)."""
    import torch
    n = a.numel()
    _expect(a, a=(a, (n,), torch.float32), b=(b, (n,), torch.float32), out_a=(out_a, (n,), torch.float32),
            out_b=(out_b, (n,), torch.float32))
    out_a = torch.empty_like(a) if out_a is None else out_a
    out_b = torch.empty_like(b) if out_b is None else out_b
    _check(_load().ssm_affine_exclusive_scan(_ptr(a), _ptr(b), _ptr(out_a), _ptr(out_b), n, _stream(stream)))
    return out_a, out_b


def ssm_ssd_plan_query(batch: int, seqlen: int, nheads: int, headdim: int = 64, ngroups: int = 1,
                       d_state: int = 128) -> dict:
    """The time chunks ``ssm_ssd_fwd`` picks for these sizes."""
    p = ssm_plan()
    _check(_load().ssm_ssd_plan_query(batch, seqlen, nheads, headdim, ngroups, d_state, ctypes.byref(p)))
    return {"chunk_len": p.chunk_len, "n_chunks": p.n_chunks}


def ssm_ssd_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus: bool = True, initial_state=None,
                out=None, last_state=None, out_dtype=None, stream=None, plan: Optional[dict] = None):
    """Mamba-2 (SSD) scan (see include/ssmscan.h).  x, z: [batch, seqlen, nheads, headdim]
    (bfloat16); dt: [batch, seqlen, nheads]; B, C: [batch, seqlen, ngroups, d_state]; A,
    dt_bias: [nheads] and D: [nheads * headdim] (float32); states [batch, nheads, headdim,
    d_state] float32.  Returns out (allocated if None, dtype ``out_dtype`` or x's).
    ``plan`` = {"chunk_len": ..} forces the time chunks (``ssm_ssd_fwd_plan``)."""
    import torch
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [batch, seqlen, nheads, headdim] and B [batch, seqlen, ngroups, d_state]")
    batch, seqlen, nheads, headdim = x.shape
    ngroups, d_state = B.shape[2], B.shape[3]
    f32, xs, bcs, st = torch.float32, tuple(x.shape), (batch, seqlen, ngroups, d_state), (batch, nheads, headdim, d_state)
    _expect(x, x=(x, xs, None), dt=(dt, (batch, seqlen, nheads), x.dtype), z=(z, xs, x.dtype), B=(B, bcs, x.dtype),
            C=(C, bcs, x.dtype), A=(A, (nheads,), f32), D=(D, (nheads * headdim,), f32),
            dt_bias=(dt_bias, (nheads,), f32), initial_state=(initial_state, st, f32), out=(out, xs, None),
            last_state=(last_state, st, f32))
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _flags(softplus, False),
            _ptr(initial_state), _ptr(out), _ptr(last_state), batch, seqlen, nheads, headdim, ngroups, d_state,
            _dtype_code(x), _dtype_code(out), _stream(stream))
    if plan is None:
        _check(_load().ssm_ssd_fwd(*args))
    else:
        p = ssm_plan()
        p.chunk_len = int(plan["chunk_len"])
        _check(_load().ssm_ssd_fwd_plan(*args, ctypes.byref(p)))
    return out


def ssm_ssd_state_update(state, x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus: bool = True, out=None,
                         out_dtype=None, stream=None):
    """One Mamba-2 decode step; ``state`` [batch, nheads, headdim, d_state] float32 is
    updated in place.  x, z: [batch, nheads, headdim]; dt: [batch, nheads]; B, C:
    [batch, ngroups, d_state].  Returns out."""
    import torch
    if x.dim() != 3 or B.dim() != 3:
        raise ValueError("x must be [batch, nheads, headdim] and B [batch, ngroups, d_state]")
    batch, nheads, headdim = x.shape
    ngroups, d_state = B.shape[1], B.shape[2]
    f32, xs, bcs = torch.float32, tuple(x.shape), (batch, ngroups, d_state)
    _expect(x, state=(state, (batch, nheads, headdim, d_state), f32), x=(x, xs, None),
            dt=(dt, (batch, nheads), x.dtype), z=(z, xs, x.dtype), B=(B, bcs, x.dtype), C=(C, bcs, x.dtype),
            A=(A, (nheads,), f32), D=(D, (nheads * headdim,), f32), dt_bias=(dt_bias, (nheads,), f32),
            out=(out, xs, None))
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    _check(_load().ssm_ssd_state_update(_ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                        _ptr(dt_bias), _flags(softplus, False), _ptr(out), batch, nheads, headdim,
                                        ngroups, d_state, _dtype_code(x), _dtype_code(out), _stream(stream)))
    return out
