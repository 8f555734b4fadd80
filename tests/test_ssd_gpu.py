"""GPU parity of the Mamba-2 (SSD) scan (ssm_ssd_fwd) and decode step
(ssm_ssd_state_update) against the fp64 oracle, through the C ABI.

Bar: bf16 inputs with fp32 state, max per-row relative error <= 2e-3 (rows:
(b, h, p) over t for out; (b, h, p) over n for the state).  The chunk products
run on bf16 matrix cores with the computed operands split into two bf16
terms, so the measured error is far below the bar; the tests also hold it to
2e-4 to catch a lost split.  bf16 out equals round-to-nearest-even of fp32 out
bitwise.  The decode step is elementwise fp32 and is held to 1e-5 (fp32
inputs) and 2e-3 (bf16 inputs).
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import rne_bf16_of, rowinf, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ssm = pytest.importorskip("sequence_scan_amd")

TOL, TIGHT = 2e-3, 2e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ssm.library()


def _dev(inp):
    tdt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    out = {}
    for k, v in inp.items():
        if k == "dtype":
            continue
        t = torch.from_numpy(np.ascontiguousarray(v))
        if k in ("x", "dt", "z", "B", "C"):
            t = t.to(tdt)  # exact: the values are representable in the input dtype
        out[k] = t.cuda()
    return out


def _case(batch, L, H, G, N, seed, dtype="bf16"):
    cfg = workloads.SsdConfig("t", batch, L, H, 64, G, N, dtype)
    return workloads.ssd_inputs(cfg, seed=seed)


def _run(inp, use=("D", "z", "dt_bias"), softplus=True, h0=None, out_dtype=torch.float32, in_place=False,
         chunk_len=None):
    t = _dev(inp)
    batch, L, H, P = inp["x"].shape
    N = inp["B"].shape[3]
    h = torch.from_numpy(h0).cuda() if h0 is not None else None
    last = h if in_place else torch.full((batch, H, P, N), float("nan"), device="cuda")
    out = ssm.ssm_ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"] if "D" in use else None,
                          t["z"] if "z" in use else None, t["dt_bias"] if "dt_bias" in use else None,
                          softplus=softplus, initial_state=h, last_state=last, out_dtype=out_dtype,
                          plan={"chunk_len": chunk_len} if chunk_len else None)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), last.cpu().numpy()


def _ref(inp, use=("D", "z", "dt_bias"), softplus=True, h0=None):
    return oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"] if "D" in use else None,
                          inp["z"] if "z" in use else None, inp["dt_bias"] if "dt_bias" in use else None,
                          softplus=softplus, h0=h0)


def _check(out, last, ref, ref_last, tol=TIGHT):
    e_out, e_last = rowinf(out, ref, 1), rowinf(last, ref_last, 3)
    print(f"  out error {e_out:.2e}, state error {e_last:.2e}")
    assert e_out <= tol and e_last <= tol


@pytest.mark.parametrize("batch,L,H,G,N", [(1, 64, 1, 1, 64), (2, 100, 3, 1, 128), (2, 257, 4, 2, 64),
                                           (1, 1, 2, 1, 128), (3, 130, 6, 3, 128), (1, 63, 2, 2, 128),
                                           (1, 1000, 2, 1, 128)])
def test_ssd_vs_oracle(batch, L, H, G, N):
    say(f"SSD batch {batch} seqlen {L} nheads {H} ngroups {G} d_state {N}")
    inp = _case(batch, L, H, G, N, seed=L + H)
    out, last = _run(inp)
    _check(out, last, *_ref(inp))


@pytest.mark.parametrize("softplus,use", [(False, ("D", "z", "dt_bias")), (True, ()), (True, ("z",)),
                                          (True, ("D",))])
def test_ssd_options(softplus, use):
    say(f"SSD options softplus={softplus} inputs={use}")
    inp = _case(2, 150, 4, 2, 128, seed=81)
    if not softplus:  # the step is used as given: draw it positive
        rng = np.random.default_rng(82)
        inp["dt"] = workloads.round_to_bf16(np.exp(rng.uniform(np.log(1e-3), np.log(0.1), inp["dt"].shape)))
        inp["dt_bias"] = np.zeros_like(inp["dt_bias"])
    out, last = _run(inp, use=use, softplus=softplus)
    _check(out, last, *_ref(inp, use=use, softplus=softplus))


@pytest.mark.parametrize("in_place", [False, True])
def test_ssd_initial_state_and_bf16_out(in_place):
    say(f"SSD from a stored state (in place {in_place}); bf16 out = RNE of fp32 out")
    inp = _case(2, 200, 3, 1, 128, seed=83)
    h0 = workloads.ssd_initial_state(2, 3, 64, 128, seed=83)
    out, last = _run(inp, h0=h0, in_place=in_place)
    _check(out, last, *_ref(inp, h0=h0))
    o16, _ = _run(inp, h0=h0, out_dtype=torch.bfloat16)
    np.testing.assert_array_equal(o16, rne_bf16_of(torch.from_numpy(out)))


def test_ssd_chunked_prefill_and_empty():
    say("SSD prefill in three pieces from the previous state; seqlen 0 copies the state")
    inp = _case(1, 300, 2, 1, 64, seed=85)
    t = _dev(inp)
    state = torch.zeros((1, 2, 64, 64), device="cuda")
    pieces = []
    for lo, hi in ((0, 70), (70, 71), (71, 300)):
        sl = {k: (v[:, lo:hi].contiguous() if k in ("x", "dt", "z", "B", "C") else v) for k, v in t.items()}
        pieces.append(ssm.ssm_ssd_fwd(sl["x"], sl["dt"], sl["A"], sl["B"], sl["C"], sl["D"], sl["z"], sl["dt_bias"],
                                      initial_state=state, last_state=state, out_dtype=torch.float32))
    torch.cuda.synchronize()
    ref, ref_last = _ref(inp)
    _check(torch.cat(pieces, dim=1).cpu().numpy(), state.cpu().numpy(), ref, ref_last)
    empty = {k: (v[:, :0].contiguous() if k in ("x", "dt", "z", "B", "C") else v) for k, v in t.items()}
    last = torch.zeros_like(state)
    ssm.ssm_ssd_fwd(empty["x"], empty["dt"], empty["A"], empty["B"], empty["C"], initial_state=state, last_state=last)
    torch.cuda.synchronize()
    assert torch.equal(last, state)


# headdim 48 at d_state 64 and 20, 40 at d_state 128 leave the second row of some
# threads (channels p and p + 256 * 4 / d_state) past the head
@pytest.mark.parametrize("dtype,P,N,G", [("f32", 64, 128, 1), ("bf16", 64, 64, 2), ("f32", 48, 64, 1),
                                         ("bf16", 20, 128, 1), ("f32", 40, 128, 2)])
def test_ssd_decode_vs_oracle(dtype, P, N, G):
    say(f"SSD decode {dtype} headdim {P} d_state {N} ngroups {G}: 5 steps from a stored state")
    batch, H, steps = 3, 4, 5
    cfg = workloads.SsdConfig("t", batch, steps, H, P, G, N, dtype)
    inp = workloads.ssd_inputs(cfg, seed=87)
    h0 = workloads.ssd_initial_state(batch, H, P, N, seed=87)
    t = _dev(inp)
    state = torch.from_numpy(h0).cuda()
    ys = []
    for s in range(steps):
        sl = {k: (v[:, s].contiguous() if k in ("x", "dt", "z", "B", "C") else v) for k, v in t.items()}
        ys.append(ssm.ssm_ssd_state_update(state, sl["x"], sl["dt"], sl["A"], sl["B"], sl["C"], sl["D"], sl["z"],
                                           sl["dt_bias"], out_dtype=torch.float32))
    torch.cuda.synchronize()
    ref, ref_last = _ref(inp, h0=h0)
    tol = 1e-5 if dtype == "f32" else TOL
    assert rowinf(torch.stack(ys, dim=1).cpu().numpy(), ref, 1) <= tol
    assert rowinf(state.cpu().numpy(), ref_last, 3) <= tol


def test_ssd_layer_shape_sampled():
    say("SSD Mamba-2-2.7B-like layer (batch 8, seqlen 2048, 80 heads x 64, d_state 128), sampled heads")
    cfg = workloads.SSD_CONFIGS["mamba2_2p7b"]
    inp = workloads.ssd_inputs(cfg, seed=0)
    out, last = _run(inp)
    sel = np.array([0, 1, 41, 79])
    sub = dict(inp)
    for k in ("x", "z", "dt"):
        sub[k] = np.ascontiguousarray(inp[k][:, :, sel])
    sub["A"] = np.ascontiguousarray(inp["A"][sel])
    sub["dt_bias"] = np.ascontiguousarray(inp["dt_bias"][sel])
    sub["D"] = np.ascontiguousarray(inp["D"].reshape(80, 64)[sel].reshape(-1))
    ref, ref_last = _ref(sub)
    _check(out[:, :, sel], last[:, sel], ref, ref_last)


# ---- time chunks (ssm_ssd_fwd_plan): pass A's end states and per-head decays,
# composed by the carry into each chunk's entering state

@pytest.mark.parametrize("batch,L,H,G,N,chunk", [(1, 200, 2, 1, 64, 32), (2, 300, 3, 1, 128, 64),
                                                 (1, 1000, 2, 2, 128, 96), (2, 257, 4, 2, 64, 128),
                                                 (1, 65, 1, 1, 128, 32)])
def test_ssd_time_chunks_vs_oracle(batch, L, H, G, N, chunk):
    # ragged last time chunks and matrix chunks; chunks of one 32-step matrix chunk
    say(f"SSD in time chunks: batch {batch} seqlen {L} nheads {H} ngroups {G} d_state {N} chunk_len {chunk}")
    inp = _case(batch, L, H, G, N, seed=L + 7 * H)
    h0 = workloads.ssd_initial_state(batch, H, 64, N, seed=L)
    out, last = _run(inp, h0=h0, chunk_len=chunk)
    _check(out, last, *_ref(inp, h0=h0))
    out0, last0 = _run(inp, chunk_len=chunk)
    _check(out0, last0, *_ref(inp))


@pytest.mark.parametrize("softplus,use,in_place", [(False, ("D", "z", "dt_bias"), False), (True, (), True),
                                                   (True, ("z",), True)])
def test_ssd_time_chunks_options(softplus, use, in_place):
    say(f"SSD in time chunks: options softplus={softplus} inputs={use} in place {in_place}; bf16 out = RNE of fp32")
    inp = _case(2, 230, 3, 1, 128, seed=87)
    if not softplus:
        rng = np.random.default_rng(88)
        inp["dt"] = workloads.round_to_bf16(np.exp(rng.uniform(np.log(1e-3), np.log(0.1), inp["dt"].shape)))
        inp["dt_bias"] = np.zeros_like(inp["dt_bias"])
    h0 = workloads.ssd_initial_state(2, 3, 64, 128, seed=89)
    out, last = _run(inp, use=use, softplus=softplus, h0=h0, in_place=in_place, chunk_len=64)
    _check(out, last, *_ref(inp, use=use, softplus=softplus, h0=h0))
    o16, _ = _run(inp, use=use, softplus=softplus, h0=h0, out_dtype=torch.bfloat16, chunk_len=64)
    np.testing.assert_array_equal(o16, rne_bf16_of(torch.from_numpy(out)))


def test_ssd_planner_chunks_a_long_sequence():
    L, H = 8192, 2   # 2 workgroups: the planner cuts the sequence
    plan = ssm.ssm_ssd_plan_query(1, L, H, 64, 1, 128)
    say(f"SSD batch 1 seqlen {L} nheads {H} d_state 128, planner's plan {plan}")
    assert plan["n_chunks"] > 1
    inp = _case(1, L, H, 1, 128, seed=91)
    out, last = _run(inp)
    _check(out, last, *_ref(inp))
