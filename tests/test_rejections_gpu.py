"""A rejected call enqueues nothing and writes nothing (include/ssmscan.h, "Errors"):
every entry point is called through the C ABI with real device buffers and one
invalid argument at a time; its outputs, filled with a sentinel beforehand, must
keep it after a device synchronisation."""
import ctypes

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ssm = pytest.importorskip("sequence_scan_amd")

SENTINEL = 7.0
F32, BF16 = ssm.SSM_F32, ssm.SSM_BF16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ssm.library()


def _p(t, byte_offset=0):
    return None if t is None else t.data_ptr() + byte_offset


def _outs(*shapes):
    return [torch.full(s, SENTINEL, device="cuda") for s in shapes]


def _untouched(*ts):
    torch.cuda.synchronize()
    for t in ts:
        assert torch.all(t == SENTINEL), "a rejected call wrote an output"


def test_scan_rejections_write_nothing():
    lib = ssm.library()
    b, L, d, n = 2, 40, 64, 16
    x = torch.randn(b, L, d, device="cuda")
    dl, z = torch.randn(b, L, d, device="cuda"), torch.randn(b, L, d, device="cuda")
    B, C = torch.randn(b, L, n, device="cuda"), torch.randn(b, L, n, device="cuda")
    A = -torch.rand(d, n, device="cuda") - 0.5
    D, bias = torch.ones(d, device="cuda"), torch.zeros(d, device="cuda")
    out, last = _outs((b, L, d), (b, d, n))

    def call(flags=1, xo=0, out_p=None, d_state=n, ind=F32, outd=F32):
        return lib.ssm_scan_fwd(_p(x, xo), _p(dl), _p(A), _p(B), _p(C), _p(D), _p(z), _p(bias), flags,
                                out_p if out_p is not None else _p(out), _p(last), b, L, d, d_state, ind, outd, None)

    cases = {"unknown step flag": dict(flags=4), "misaligned x": dict(xo=4), "out on x": dict(out_p=_p(x)),
             "d_state 8": dict(d_state=8), "unknown dtype": dict(ind=7)}
    for name, kw in cases.items():
        say(f"rejection: ssm_scan_fwd, {name}")
        assert call(**kw) != ssm.SSM_OK, name
        _untouched(out, last)
    # the bwd rejects the ZOH coefficient
    g = _outs((b, L, d), (b, L, d), (d, n), (b, L, n), (b, L, n), (d,), (b, L, d), (d,))
    say("rejection: ssm_scan_bwd with SSM_ZOH")
    rc = lib.ssm_scan_bwd(_p(x), _p(dl), _p(A), _p(B), _p(C), _p(D), _p(z), _p(bias), ssm.SSM_ZOH, None, _p(x), None,
                          *[_p(t) for t in g], None, b, L, d, n, F32, F32, None)
    assert rc != ssm.SSM_OK
    _untouched(*g)
    # a backward plan that cuts the sequence off a tile boundary
    plan = ssm.ssm_plan()
    plan.states_per_wave, plan.chunk_len = 4, 12
    say("rejection: ssm_scan_bwd_plan with chunk_len 12")
    rc = lib.ssm_scan_bwd_plan(_p(x), _p(dl), _p(A), _p(B), _p(C), _p(D), _p(z), _p(bias), 1, None, _p(x), None,
                               *[_p(t) for t in g], None, b, L, d, n, F32, F32, None, ctypes.byref(plan))
    assert rc == ssm.SSM_ERR_UNSUPPORTED
    _untouched(*g)


def test_decode_conv_and_ssd_rejections_write_nothing():
    lib = ssm.library()
    b, d, n = 3, 64, 16
    st, out = _outs((b, d, n), (b, d))
    x = torch.randn(b, d, device="cuda")
    A = -torch.rand(d, n, device="cuda") - 0.5
    Bv = torch.randn(b, n, device="cuda")
    say("rejection: ssm_state_update, d_state 32")
    assert lib.ssm_state_update(_p(st), _p(x), _p(x), _p(A), _p(Bv), _p(Bv), None, None, None, 1, _p(out),
                                b, d, 32, F32, F32, None) != ssm.SSM_OK
    _untouched(st, out)
    say("rejection: ssm_state_update, out overlapping the state")
    assert lib.ssm_state_update(_p(st), _p(x), _p(x), _p(A), _p(Bv), _p(Bv), None, None, None, 1, _p(st, 256),
                                b, d, n, F32, F32, None) != ssm.SSM_OK
    _untouched(st, out)

    L, K = 20, 4
    xc = torch.randn(b, L, d, device="cuda")
    w = torch.randn(d, K, device="cuda")
    cout, cache = _outs((b, L, d), (b, d, K))
    say("rejection: ssm_conv1d_fwd, d_conv 5")
    assert lib.ssm_conv1d_fwd(_p(xc), _p(w), None, 1, None, _p(cout), _p(cache), b, L, d, 5, F32, F32,
                              None) != ssm.SSM_OK
    _untouched(cout, cache)
    say("rejection: ssm_conv1d_update, cache overlapping x")
    assert lib.ssm_conv1d_update(_p(cache), _p(cache, 16), _p(w), None, 1, _p(out), b, d, K, F32, F32,
                                 None) != ssm.SSM_OK
    _untouched(cache, out)

    H, P, N2 = 2, 64, 64
    xs = torch.randn(b, L, H, P, device="cuda")
    dts = torch.randn(b, L, H, device="cuda")
    Bs = torch.randn(b, L, 1, N2, device="cuda")
    As = -torch.rand(H, device="cuda")
    sout, slast = _outs((b, L, H, P), (b, H, P, N2))
    say("rejection: ssm_ssd_fwd with fp32 inputs")
    assert lib.ssm_ssd_fwd(_p(xs), _p(dts), _p(As), _p(Bs), _p(Bs), None, None, None, 1, None, _p(sout), _p(slast),
                           b, L, H, P, 1, N2, F32, F32, None) != ssm.SSM_OK
    _untouched(sout, slast)


def test_workspace_allocation_failure_writes_nothing():
    """A chunked plan whose carry workspace (65535 rows x 2 chunks x 65536 channels x
    68 bytes, about 584 GB) exceeds the device's memory: its allocation fails, the call
    returns SSM_ERR_HIP before enqueuing anything, and the next valid call succeeds (the
    failure is not reported a second time).  The tensors are never touched on this path,
    so only `out` is a real buffer (a sentinel far smaller than its nominal size); the
    inputs are distinct addresses 1 TiB apart."""
    lib = ssm.library()
    out = torch.full((4096,), SENTINEL, device="cuda")
    base, G = out.data_ptr(), 1 << 40
    batch, L, Dn = 65535, 2, 65536
    plan = ssm.ssm_plan()
    plan.states_per_wave, plan.chunk_len = 4, 1
    say("scan whose carry workspace cannot be allocated")
    st = lib.ssm_scan_fwd_plan(base + G, base + 2 * G, base + 3 * G, base + 4 * G, base + 5 * G, None, None, None, 1,
                               base, None, batch, L, Dn, 16, BF16, F32, None, ctypes.byref(plan))
    assert st == ssm.SSM_ERR_HIP, (st, ssm.ssm_last_error())
    assert "workspace allocation" in ssm.ssm_last_error()
    _untouched(out)
    say("a valid chunked scan right after the failed one")
    x = torch.randn(1, 64, 64, device="cuda")
    B, C = torch.randn(1, 64, 16, device="cuda"), torch.randn(1, 64, 16, device="cuda")
    A = -torch.rand(64, 16, device="cuda") - 0.5
    y = ssm.ssm_scan_fwd(x, torch.randn(1, 64, 64, device="cuda"), A, B, C, plan={"states_per_wave": 4, "chunk_len": 8})
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(y))
