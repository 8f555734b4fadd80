"""GPU parity of the scan continued from a stored state (ssm_scan_fwd_from)
against the fp64 oracle, through the C ABI.

Bars as for the scan: per-row relative error <= 1e-5 with fp32 inputs and
<= 2e-3 with bf16 inputs (fp32 state).
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import rowinf, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ssm = pytest.importorskip("sequence_scan_amd")

TOL_F32, TOL_BF16 = 1e-5, 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ssm.library()


def _case(dtype, batch, L, Dn, seed):
    cfg = workloads.ScanConfig("small", batch, Dn, 16, L, dtype)
    inp = workloads.scan_inputs(cfg, seed=seed, random_params=True)
    h0 = workloads.initial_state(batch, Dn, seed=seed)
    return inp, h0


def _run_from(inp, h0, plan=None, in_place=False):
    t = to_dev(inp)
    batch, L, Dn = inp["x"].shape
    h = torch.from_numpy(h0).cuda() if h0 is not None else None
    last = h if in_place else torch.full((batch, Dn, 16), float("nan"), device="cuda")
    out = ssm.ssm_scan_fwd_from(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                                initial_state=h, last_state=last, out_dtype=torch.float32, plan=plan)
    torch.cuda.synchronize()
    return out.cpu().numpy(), last.cpu().numpy()


def _ref(inp, h0):
    return oracle.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                           inp["delta_bias"], h0=h0)


@pytest.mark.parametrize("plan", [None, {"states_per_wave": 4, "chunk_len": 37}, {"states_per_wave": 2, "chunk_len": 300},
                                  {"states_per_wave": 16, "chunk_len": 64}, {"states_per_wave": 1, "chunk_len": 129}])
@pytest.mark.parametrize("in_place", [False, True])
def test_scan_from_state_vs_oracle(plan, in_place):
    say(f"scan from a stored state, plan {plan}, in place {in_place}")
    inp, h0 = _case("f32", 2, 300, 200, seed=31)
    out, last = _run_from(inp, h0, plan=plan, in_place=in_place)
    ref, ref_last = _ref(inp, h0)
    assert rowinf(out, ref, 1) <= TOL_F32
    assert rowinf(last, ref_last, 2) <= TOL_F32


def test_scan_from_state_bf16():
    say("scan from a stored state, bf16 inputs")
    inp, h0 = _case("bf16", 3, 257, 130, seed=33)
    out, last = _run_from(inp, h0)
    ref, ref_last = _ref(inp, h0)
    assert rowinf(out, ref, 1) <= TOL_BF16
    assert rowinf(last, ref_last, 2) <= TOL_BF16


def test_chunked_prefill_equals_one_scan():
    say("prefill in three pieces, each from the previous final state, equals one scan")
    inp, _ = _case("bf16", 2, 600, 320, seed=35)
    t = to_dev(inp)
    full = ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                            out_dtype=torch.float32)
    state = torch.zeros((2, 320, 16), device="cuda")
    pieces = []
    for lo, hi in ((0, 250), (250, 251), (251, 600)):
        sl = {k: (v[:, lo:hi].contiguous() if k in ("x", "delta", "z", "B", "C") else v) for k, v in t.items()}
        pieces.append(ssm.ssm_scan_fwd_from(sl["x"], sl["delta"], sl["A"], sl["B"], sl["C"], sl["D"], sl["z"],
                                            sl["delta_bias"], initial_state=state, last_state=state,
                                            out_dtype=torch.float32))
    torch.cuda.synchronize()
    joined = torch.cat(pieces, dim=1).cpu().numpy()
    assert rowinf(joined, full.cpu().numpy(), 1) <= 1e-5
    ref, ref_last = _ref(inp, None)
    assert rowinf(state.cpu().numpy(), ref_last, 2) <= TOL_BF16


def test_empty_continuation_copies_the_state():
    say("scan from a stored state with seqlen 0")
    inp, h0 = _case("f32", 2, 0, 64, seed=37)
    t = to_dev(inp)
    h = torch.from_numpy(h0).cuda()
    last = torch.zeros_like(h)
    ssm.ssm_scan_fwd_from(t["x"], t["delta"], t["A"], t["B"], t["C"], initial_state=h, last_state=last)
    torch.cuda.synchronize()
    assert torch.equal(last, h)


def test_long_sequence_from_state_sampled():
    say("long DNA-like sequence (batch 1, d_inner 2048, L 262144) from a stored state, sampled channels")
    cfg = workloads.SCAN_CONFIGS["long_dna"]
    inp = workloads.scan_inputs(cfg, seed=1)
    h0 = workloads.initial_state(cfg.batch, cfg.d_inner, seed=1)
    out, last = _run_from(inp, h0)
    sel = np.array([0, 63, 64, 1000, 2047])
    sub = dict(inp)
    for k in ("x", "delta", "z"):
        sub[k] = np.ascontiguousarray(inp[k][..., sel])
    for k in ("A", "D", "delta_bias"):
        sub[k] = np.ascontiguousarray(inp[k][sel])
    ref, ref_last = _ref(sub, np.ascontiguousarray(h0[:, sel]))
    assert rowinf(out[..., sel], ref, 1) <= TOL_BF16
    assert rowinf(last[:, sel], ref_last, 2) <= TOL_BF16
