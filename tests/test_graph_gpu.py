"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Each call enqueues only kernels on the caller's stream (the state copies and
zero fills are kernels, not memset or memcpy nodes), so it can be captured.
Every replay must reproduce the eager result bit for bit; the replays are
separated by eager work on the same buffers and by synchronisations.
"""
import numpy as np
import pytest

import workloads
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ssm = pytest.importorskip("sequence_scan_amd")

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ssm.library()


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(g, reset, outputs, expected):
    """Replay REPLAYS times; before each, `reset` restores the inputs the graph
    updates in place and poisons its outputs (eager work), then compares."""
    for r in range(REPLAYS):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("out", "state"), outputs, expected):
            assert torch.equal(got, want), f"replay {r}: {name} differs from the eager result"


def _poison(*ts):
    for t in ts:
        t.fill_(float("nan"))


@pytest.mark.parametrize("chunk_len", [None, 96])
def test_scan_graph(chunk_len):
    L = 300
    say(f"graph: scan batch 2 L {L} d_inner 200 bf16, chunk_len {chunk_len}")
    cfg = workloads.ScanConfig("g", 2, 200, 16, L, "bf16")
    t = to_dev(workloads.scan_inputs(cfg, seed=21))
    plan = {"states_per_wave": 4, "chunk_len": chunk_len} if chunk_len else None
    out = torch.empty((2, L, 200), device="cuda")
    last = torch.empty((2, 200, 16), device="cuda")

    def call():
        ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                         out=out, last_state=last, plan=plan)

    call()
    torch.cuda.synchronize()
    want = (out.clone(), last.clone())
    g = _capture(call)
    _replay_and_check(g, lambda: _poison(out, last), (out, last), want)


def test_decode_steps_graph():
    steps = 12
    say(f"graph: {steps} decode steps batch 4 d_inner 300 bf16")
    cfg = workloads.DecodeConfig("g", 4, 300, 16, steps, "bf16")
    t = to_dev(workloads.decode_inputs(cfg, seed=22, random_params=True))
    state0 = torch.randn((4, 300, 16), generator=torch.Generator().manual_seed(3)).cuda()
    state = state0.clone()
    out = torch.empty((steps, 4, 300), device="cuda")

    def call():
        for s in range(steps):
            ssm.ssm_state_update(state, t["x"][s], t["delta"][s], t["A"], t["B"][s], t["C"][s], t["D"],
                                 t["z"][s], t["delta_bias"], softplus=True, out=out[s])

    call()
    torch.cuda.synchronize()
    want = (out.clone(), state.clone())
    state.copy_(state0)
    g = _capture(call)  # the warm-up advanced the state; the reset below restores it

    def reset():
        state.copy_(state0)
        _poison(out)

    _replay_and_check(g, reset, (out, state), want)


def test_conv1d_graph():
    say("graph: conv1d prefill + cache, then 4 decode steps, batch 2 L 70 d_inner 96 bf16")
    inp = workloads.conv_inputs(2, 70, 96, 4, "bf16", seed=23, with_state=True)
    x = torch.from_numpy(inp["x"]).to(torch.bfloat16).cuda()
    w = torch.from_numpy(inp["weight"]).cuda()
    b = torch.from_numpy(inp["bias"]).cuda()
    st0 = torch.from_numpy(inp["conv_state"]).to(torch.bfloat16).cuda()
    xs = torch.randn((4, 2, 96), generator=torch.Generator().manual_seed(4)).to(torch.bfloat16).cuda()
    out = torch.empty_like(x)
    cache = torch.empty_like(st0)
    yd = torch.empty((4, 2, 96), dtype=torch.bfloat16, device="cuda")

    def call():
        ssm.ssm_conv1d_fwd(x, w, b, conv_state_in=st0, out=out, conv_state_out=cache)
        for s in range(4):
            ssm.ssm_conv1d_update(cache, xs[s], w, b, out=yd[s])

    call()
    torch.cuda.synchronize()
    want = (torch.cat([out.flatten(), yd.flatten()]), cache.clone())
    g = _capture(call)

    def reset():
        out.fill_(0)
        yd.fill_(0)
        cache.fill_(0)

    for r in range(REPLAYS):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.cat([out.flatten(), yd.flatten()]), want[0]), f"replay {r}: outputs differ"
        assert torch.equal(cache, want[1]), f"replay {r}: cache differs"


@pytest.mark.parametrize("chunk_len", [None, 32])
def test_ssd_graph(chunk_len):
    say(f"graph: Mamba-2 SSD batch 2 L 100 heads 4 x 64 d_state 64 bf16 (chunk_len {chunk_len}), then 3 decode steps")
    cfg = workloads.SsdConfig("g", 2, 100, 4, 64, 1, 64)
    t = {k: (torch.from_numpy(v).to(torch.bfloat16) if k in ("x", "dt", "z", "B", "C") else torch.from_numpy(v)).cuda()
         for k, v in workloads.ssd_inputs(cfg, seed=24).items() if k != "dtype"}
    out = torch.empty(t["x"].shape, device="cuda")
    last = torch.empty((2, 4, 64, 64), device="cuda")
    yd = torch.empty((3, 2, 4, 64), device="cuda")
    # the decode steps take the first three steps' inputs again, as [batch, ...] tensors
    dec = [{k: t[k][:, s].contiguous() for k in ("x", "dt", "z", "B", "C")} for s in range(3)]

    def call():
        ssm.ssm_ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["z"], t["dt_bias"],
                        out=out, last_state=last, plan={"chunk_len": chunk_len} if chunk_len else None)
        for s, d in enumerate(dec):
            ssm.ssm_ssd_state_update(last, d["x"], d["dt"], t["A"], d["B"], d["C"], t["D"], d["z"], t["dt_bias"],
                                     softplus=True, out=yd[s])

    call()
    torch.cuda.synchronize()
    want = (torch.cat([out.flatten(), yd.flatten()]), last.clone())
    g = _capture(call)
    for r in range(REPLAYS):
        _poison(out, yd, last)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.cat([out.flatten(), yd.flatten()]), want[0]), f"replay {r}: outputs differ"
        assert torch.equal(last, want[1]), f"replay {r}: state differs"
    assert np.isfinite(want[0].cpu().numpy()).all()


@pytest.mark.parametrize("chunk_len", [None, 32])
def test_backward_graph(chunk_len):
    """The backward, whose workspace comes from hipMallocAsync on the capturing
    stream (a graph allocation node; outside capture it comes from the library's
    pool), one chunk and time chunks (forward and reverse carries)."""
    L = 150
    say(f"graph: backward batch 2 L {L} d_inner 96 bf16, chunk_len {chunk_len}")
    cfg = workloads.ScanConfig("g", 2, 96, 16, L, "bf16")
    t = to_dev(workloads.scan_inputs(cfg, seed=25, random_params=True))
    gen = torch.Generator().manual_seed(6)
    dout = torch.randn((2, L, 96), generator=gen).cuda()
    dlast = torch.randn((2, 96, 16), generator=gen).cuda()
    h0 = torch.randn((2, 96, 16), generator=gen).cuda()
    plan = {"states_per_wave": 4, "chunk_len": chunk_len} if chunk_len else None
    outs = {}

    def call():
        outs.update(ssm.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                                     softplus=True, initial_state=h0, dout=dout, dlast_state=dlast,
                                     want_dinitial_state=True, plan=plan))

    call()
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in outs.items()}
    g = _capture(call)  # the capture's call allocated the gradients that replays write
    for r in range(REPLAYS):
        _poison(*outs.values())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v, want[k]), f"replay {r}: {k} differs from the eager result"
