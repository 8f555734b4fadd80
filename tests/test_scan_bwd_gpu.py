"""GPU parity of the scan's backward (ssm_scan_bwd) against the fp64 oracle,
through the C ABI.

Bar: the inputs are identical on both sides, so fp32 rounding is all that
separates them.  The backward runs the recurrence twice (forward, then the
reverse adjoint) and sums long products, so its bar is 1e-4 per-row relative
error (rows: (b, d) over t for dx, ddelta, dz; (b, n) over t for dB, dC; d over
n for dA; (b, d) over n for the initial state's gradient), with whole-vector
relative error for dD and ddelta_bias; measured errors are about 1e-6.  bf16
gradients equal round-to-nearest-even of the fp32 gradients bitwise.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import rne_bf16_of, rowinf, say, slice_channels, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ssm = pytest.importorskip("sequence_scan_amd")

TOL = 1e-4
AXES = {"dx": 1, "ddelta": 1, "dz": 1, "dB": 1, "dC": 1, "dA": 1, "dinitial_state": 2, "dh0": 2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ssm.library()


def _case(batch, L, Dn, dtype="f32", seed=3, softplus=True):
    cfg = workloads.ScanConfig("small", batch, Dn, 16, L, dtype)
    inp = workloads.scan_inputs(cfg, seed=seed, random_params=True)
    rng = np.random.default_rng(seed + 100)
    if not softplus:  # the step is used as given: draw it positive
        inp["delta"] = workloads.round_to_bf16(np.exp(rng.uniform(np.log(1e-3), np.log(0.1), inp["delta"].shape)))
        inp["delta_bias"] = rng.uniform(0.0, 0.01, Dn).astype(np.float32)
    g = workloads.round_to_bf16(rng.standard_normal((batch, L, Dn)).astype(np.float32))  # exact in bf16 and fp32
    gl = rng.standard_normal((batch, Dn, 16)).astype(np.float32)
    h0 = workloads.initial_state(batch, Dn, seed=seed)
    return inp, g, gl, h0


def _run(inp, g, gl, h0, softplus=True, use=("D", "z", "delta_bias"), grad_dtype=torch.float32):
    t = to_dev(inp)
    dout = torch.from_numpy(g).to(grad_dtype).cuda()
    res = ssm.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"] if "D" in use else None,
                           t["z"] if "z" in use else None, t["delta_bias"] if "delta_bias" in use else None,
                           softplus=softplus, initial_state=torch.from_numpy(h0).cuda() if h0 is not None else None,
                           dout=dout, dlast_state=torch.from_numpy(gl).cuda() if gl is not None else None,
                           want_dinitial_state=True)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy() for k, v in res.items()}


def _ref(inp, g, gl, h0, softplus=True, use=("D", "z", "delta_bias")):
    return oracle.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"] if "D" in use else None,
                           inp["z"] if "z" in use else None, inp["delta_bias"] if "delta_bias" in use else None,
                           softplus=softplus, h0=h0, dout=g, dlast=gl)


def _compare(got, ref, tol=TOL):
    ref = dict(ref)
    if "dh0" in ref:
        ref["dinitial_state"] = ref.pop("dh0")
    for k, r in ref.items():
        if k in AXES:
            err = rowinf(got[k], r, AXES[k])
        else:
            err = float(np.max(np.abs(got[k] - r)) / max(1e-30, float(np.max(np.abs(r)))))
        assert err <= tol, f"{k}: {err:.3e}"


@pytest.mark.parametrize("batch,L,Dn", [(1, 40, 64), (2, 37, 70), (2, 300, 200), (1, 5, 8), (3, 129, 256)])
def test_bwd_vs_oracle(batch, L, Dn):
    say(f"backward batch {batch} seqlen {L} d_inner {Dn}")
    inp, g, gl, h0 = _case(batch, L, Dn)
    _compare(_run(inp, g, gl, h0), _ref(inp, g, gl, h0))


@pytest.mark.parametrize("softplus,use", [(False, ("D", "z", "delta_bias")), (True, ()), (True, ("z",)),
                                          (True, ("D", "delta_bias"))])
def test_bwd_options(softplus, use):
    say(f"backward options softplus={softplus} inputs={use}")
    inp, g, gl, h0 = _case(2, 70, 96, softplus=softplus, seed=7)
    got = _run(inp, g, None, None, softplus=softplus, use=use)
    ref = _ref(inp, g, None, None, softplus=softplus, use=use)
    _compare(got, ref)
    # the initial state's gradient does not depend on the initial state's value
    ref0 = _ref(inp, g, None, np.zeros_like(h0), softplus=softplus, use=use)
    assert rowinf(got["dinitial_state"], ref0["dh0"], 2) <= TOL


def test_bwd_bf16_inputs_and_gradients():
    say("backward with bf16 inputs: fp32 gradients vs the oracle, bf16 gradients = RNE of fp32")
    inp, g, gl, h0 = _case(2, 100, 128, dtype="bf16", seed=9)
    g32 = _run(inp, g, gl, h0)
    _compare(g32, _ref(inp, g, gl, h0))
    g16 = _run(inp, g, gl, h0, grad_dtype=torch.bfloat16)
    for k in ("dx", "ddelta", "dz", "dB", "dC"):
        np.testing.assert_array_equal(g16[k], rne_bf16_of(torch.from_numpy(g32[k])), err_msg=k)
    for k in ("dA", "dD", "ddelta_bias", "dinitial_state"):
        np.testing.assert_array_equal(g16[k], g32[k], err_msg=k)


def test_bwd_deterministic_and_empty():
    say("backward determinism; seqlen 0")
    inp, g, gl, h0 = _case(2, 45, 130, seed=11)
    a = _run(inp, g, gl, h0)
    b = _run(inp, g, gl, h0)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    inp0, g0, gl0, h00 = _case(2, 0, 64, seed=12)
    got = _run(inp0, g0, gl0, h00)
    assert not np.any(got["dA"]) and not np.any(got["dD"]) and not np.any(got["ddelta_bias"])
    np.testing.assert_array_equal(got["dinitial_state"], gl0)


def test_bwd_layer_shape():
    say("backward, Mamba-2.8B-like layer at batch 1 (all channels: dB, dC) and batch 8 (sampled channels)")
    cfg = workloads.SCAN_CONFIGS["mamba2p8b"]
    inp = workloads.scan_inputs(cfg, seed=0, batch=1)
    rng = np.random.default_rng(5)
    g = workloads.round_to_bf16(rng.standard_normal(inp["x"].shape).astype(np.float32))
    got = _run(inp, g, None, None)
    ref = _ref(inp, g, None, None)
    _compare(got, ref)
    inp8 = workloads.scan_inputs(cfg, seed=0)
    g8 = workloads.round_to_bf16(rng.standard_normal(inp8["x"].shape).astype(np.float32))
    got8 = _run(inp8, g8, None, None)
    sel = np.array([0, 63, 64, 2500, 5119])
    sub = slice_channels(inp8, sel)
    ref8 = _ref(sub, np.ascontiguousarray(g8[..., sel]), None, None)
    for k in ("dx", "ddelta", "dz"):
        assert rowinf(got8[k][..., sel], ref8[k], 1) <= TOL, k
    assert rowinf(got8["dA"][sel], ref8["dA"], 1) <= TOL
    for k in ("dD", "ddelta_bias"):
        err = float(np.max(np.abs(got8[k][sel] - ref8[k])) / np.max(np.abs(ref8[k])))
        assert err <= TOL, k
