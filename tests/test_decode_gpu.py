"""GPU parity of the decode step (ssm_state_update) against the oracle and the scan."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import rowinf, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ssm = pytest.importorskip("sequence_scan_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ssm.library()


def _decode_run(t, steps, state, out_dtype=torch.float32):
    ys = []
    for s in range(steps):
        ys.append(ssm.ssm_state_update(state, t["x"][s], t["delta"][s], t["A"], t["B"][s], t["C"][s], t["D"],
                                       t["z"][s], t["delta_bias"], softplus=True, out_dtype=out_dtype))
    torch.cuda.synchronize()
    return torch.stack(ys).float().cpu().numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_vs_oracle(dtype):
    say(f"decode {dtype} 24 steps batch 3 d_inner 200")
    cfg = workloads.DecodeConfig("d", 3, 200, 16, 24, dtype)
    inp = workloads.decode_inputs(cfg, seed=5, random_params=True)
    t = to_dev(inp)
    state = torch.zeros((3, 200, 16), device="cuda")
    y = _decode_run(t, 24, state)
    st = np.zeros((3, 200, 16))
    ref = []
    for s in range(24):
        r, st = oracle.state_update(st, inp["x"][s], inp["delta"][s], inp["A"], inp["B"][s], inp["C"][s],
                                    inp["D"], inp["z"][s], inp["delta_bias"])
        ref.append(r)
    ref = np.stack(ref)
    tol = 1e-5 if dtype == "f32" else 2e-3
    assert rowinf(y, ref, 0) <= tol            # rows (b, d) over steps
    assert rowinf(state.cpu().numpy(), st, 2) <= tol


def test_decode_equals_scan_and_prefill_continuation():
    say("decode steps == scan; prefill + decode == scan")
    cfg = workloads.DecodeConfig("d", 2, 130, 16, 40, "f32")
    inp = workloads.decode_inputs(cfg, seed=6, random_params=True)
    t = to_dev(inp)
    # scan layout [batch, L, ...]
    sc = {k: (t[k].transpose(0, 1).contiguous() if k in ("x", "delta", "z", "B", "C") else t[k]) for k in t}
    last = torch.empty((2, 130, 16), device="cuda")
    yscan = ssm.ssm_scan_fwd(sc["x"], sc["delta"], sc["A"], sc["B"], sc["C"], sc["D"], sc["z"], sc["delta_bias"],
                             last_state=last, plan={"states_per_wave": 4, "chunk_len": 16})
    state = torch.zeros((2, 130, 16), device="cuda")
    ydec = _decode_run(t, 40, state)
    ys = yscan.transpose(0, 1).cpu().numpy()
    assert rowinf(ydec, ys, 0) <= 1e-5
    assert rowinf(state.cpu().numpy(), last.cpu().numpy(), 2) <= 1e-5
    # prefill the first 25 steps, then decode 15 more from its final state
    L1 = 25
    st1 = torch.empty((2, 130, 16), device="cuda")
    ssm.ssm_scan_fwd(sc["x"][:, :L1].contiguous(), sc["delta"][:, :L1].contiguous(), sc["A"],
                     sc["B"][:, :L1].contiguous(), sc["C"][:, :L1].contiguous(), sc["D"],
                     sc["z"][:, :L1].contiguous(), sc["delta_bias"], last_state=st1)
    rest = {k: (v[L1:] if k in ("x", "delta", "z", "B", "C") else v) for k, v in t.items()}
    y2 = _decode_run(rest, 40 - L1, st1)
    assert rowinf(y2, ys[L1:], 0) <= 1e-5
    assert rowinf(st1.cpu().numpy(), last.cpu().numpy(), 2) <= 1e-5
