"""The scan entry point that allocates nothing (ssm_scan_fwd_noalloc), through the
C ABI, against the allocating entry point it varies (ssm_scan_fwd_from) and the
oracle.

Both run the same kernels on the same plan; only the carry workspace differs (a
fixed per-device array instead of a stream-ordered allocation), so the results
must agree bit for bit, and with the oracle to the usual bars (1e-5 for fp32
inputs, 2e-3 for bf16).  Calls run back to back with the second smaller than the
first, so stale scratch contents from the first call would show in the second.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import Parity, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ssm = pytest.importorskip("sequence_scan_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ssm.library()


def _case(dtype, batch, seqlen, d_inner, seed):
    cfg = workloads.ScanConfig("noalloc", batch, d_inner, 16, seqlen, dtype)
    inp = workloads.scan_inputs(cfg, seed=seed, random_params=True)
    h0 = workloads.initial_state(batch, d_inner, 16, seed=seed)
    return inp, h0


def _call(fn, t, h0, plan, in_place):
    bsz, L, Dn = t["x"].shape
    out = torch.full((bsz, L, Dn), float("nan"), device="cuda")
    st = torch.from_numpy(h0).cuda()
    if in_place:
        last = st
    else:
        last = torch.full((bsz, Dn, 16), float("nan"), device="cuda")
    fn(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], softplus=True,
       initial_state=st, out=out, last_state=last, plan=plan)
    return out, last


CASES = [
    # (dtype, batch, seqlen, d_inner, chunk_len, state in place)
    ("bf16", 2, 3000, 384, 512, False),    # 6 chunks
    ("f32", 1, 700, 130, 100, True),       # 7 chunks, smaller, initial state replaced in place
]


def test_noalloc_matches_the_allocating_call():
    results = []
    for i, (dtype, bsz, L, Dn, chunk, in_place) in enumerate(CASES):
        say(f"noalloc call {i}: {dtype} batch {bsz} seqlen {L} d_inner {Dn} chunk {chunk} in_place {in_place}")
        inp, h0 = _case(dtype, bsz, L, Dn, seed=40 + i)
        t = to_dev(inp)
        plan = {"states_per_wave": 4, "chunk_len": chunk}
        out, last = _call(ssm.ssm_scan_fwd_noalloc, t, h0, plan, in_place)
        results.append((inp, h0, t, plan, in_place, out, last))
    torch.cuda.synchronize()
    for i, (inp, h0, t, plan, in_place, out, last) in enumerate(results):
        say(f"noalloc call {i}: against ssm_scan_fwd_from and the oracle")
        ref_out, ref_last = _call(ssm.ssm_scan_fwd_from, t, h0, plan, in_place)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"call {i}: out differs from the allocating call"
        assert torch.equal(last, ref_last), f"call {i}: last_state differs from the allocating call"
        o, o_last = oracle.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                    inp["delta_bias"], softplus=True, h0=h0)
        bar = 1e-5 if inp["dtype"] == "f32" else 2e-3
        po = Parity(f"noalloc call {i} out")
        for b in range(o.shape[0]):
            po.add(out[b].cpu().numpy(), o[b], axis=0)
        po.check(bar)
        Parity(f"noalloc call {i} last_state").add(last.cpu().numpy(), o_last, axis=2).check(bar)


def test_noalloc_long_sequence_default_plan():
    """One row of 65536 steps over 2048 channels: the planner cuts it into time chunks
    whose carry workspace (about 9 MB) sits in the fixed scratch."""
    cfg = workloads.SCAN_CONFIGS["long_dna"]
    bsz, L, Dn = 1, 65536, cfg.d_inner
    plan = ssm.ssm_scan_plan(bsz, L, Dn)
    assert plan["n_chunks"] > 1
    say(f"noalloc long row: batch {bsz} seqlen {L} d_inner {Dn}, default plan {plan}")
    inp = workloads.scan_inputs(cfg, seed=3, seqlen=L)
    t = to_dev(inp)
    h0 = np.zeros((bsz, Dn, 16), dtype=np.float32)
    out, last = _call(ssm.ssm_scan_fwd_noalloc, t, h0, None, False)
    ref_out, ref_last = _call(ssm.ssm_scan_fwd_from, t, h0, None, False)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(last, ref_last)
