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


def _run(inp, g, gl, h0, softplus=True, use=("D", "z", "delta_bias"), grad_dtype=torch.float32, chunk_len=None):
    t = to_dev(inp)
    dout = torch.from_numpy(g).to(grad_dtype).cuda()
    res = ssm.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"] if "D" in use else None,
                           t["z"] if "z" in use else None, t["delta_bias"] if "delta_bias" in use else None,
                           softplus=softplus, initial_state=torch.from_numpy(h0).cuda() if h0 is not None else None,
                           dout=dout, dlast_state=torch.from_numpy(gl).cuda() if gl is not None else None,
                           want_dinitial_state=True,
                           plan={"states_per_wave": 4, "chunk_len": chunk_len} if chunk_len else None)
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
    # batch 1 has 80 channel blocks, which the planner cuts into time chunks; batch 8 runs in one chunk
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


# ---- time-chunked backward (ssm_scan_bwd_plan): each chunk starts from the state
# the forward carry gives it and from the gradient the reverse carry gives it

@pytest.mark.parametrize("batch,L,Dn,chunk", [(1, 100, 64, 16), (2, 203, 70, 24), (1, 77, 65, 8), (2, 300, 200, 64),
                                              (1, 1000, 128, 104)])
def test_bwd_chunked_vs_oracle(batch, L, Dn, chunk):
    # ragged last chunks and tiles; an odd d_inner (one-channel items); chunks of one tile
    say(f"chunked backward batch {batch} seqlen {L} d_inner {Dn} chunk_len {chunk}")
    inp, g, gl, h0 = _case(batch, L, Dn, seed=13)
    _compare(_run(inp, g, gl, h0, chunk_len=chunk), _ref(inp, g, gl, h0))


@pytest.mark.parametrize("softplus,use", [(False, ("D", "z", "delta_bias")), (True, ()), (True, ("z",))])
def test_bwd_chunked_options(softplus, use):
    say(f"chunked backward options softplus={softplus} inputs={use}")
    inp, g, gl, h0 = _case(2, 150, 96, softplus=softplus, seed=17)
    _compare(_run(inp, g, None, None, softplus=softplus, use=use, chunk_len=32),
             _ref(inp, g, None, None, softplus=softplus, use=use))
    _compare(_run(inp, g, gl, h0, softplus=softplus, use=use, chunk_len=40),
             _ref(inp, g, gl, h0, softplus=softplus, use=use))


def test_bwd_chunked_bf16_and_deterministic():
    say("chunked backward with bf16 inputs: fp32 gradients vs the oracle, bf16 = RNE of fp32, repeat is bitwise equal")
    inp, g, gl, h0 = _case(2, 200, 128, dtype="bf16", seed=19)
    g32 = _run(inp, g, gl, h0, chunk_len=48)
    _compare(g32, _ref(inp, g, gl, h0))
    again = _run(inp, g, gl, h0, chunk_len=48)
    for k in g32:
        assert np.array_equal(g32[k], again[k]), k
    g16 = _run(inp, g, gl, h0, grad_dtype=torch.bfloat16, chunk_len=48)
    for k in ("dx", "ddelta", "dz", "dB", "dC"):
        np.testing.assert_array_equal(g16[k], rne_bf16_of(torch.from_numpy(g32[k])), err_msg=k)


def test_bwd_planner_chunks_a_long_sequence():
    L, Dn = 16384, 256  # 4 channel blocks: the planner cuts the sequence
    plan = ssm.ssm_scan_bwd_plan_query(1, L, Dn)
    say(f"backward, batch 1 seqlen {L} d_inner {Dn} bf16, planner's plan {plan}")
    assert plan["n_chunks"] > 1
    inp, g, gl, h0 = _case(1, L, Dn, dtype="bf16", seed=21)
    _compare(_run(inp, g, gl, h0), _ref(inp, g, gl, h0))


def test_bwd_long_dna_sampled():
    """The long single-row workload (batch 1, seqlen 262144, d_inner 2048) on the
    planner's chunks, inputs drawn on the GPU.  Per-channel gradients are checked on
    sampled channels over the whole sequence (a channel's gradients depend on no
    other channel).  dB and dC sum over all channels: dB of the last steps depends
    only on those steps (the reverse walk starts at the end, with no dlast), and dC
    of the first steps only on the first steps (the forward starts from zero), so
    both are checked there against the oracle run on those steps alone."""
    cfg = workloads.SCAN_CONFIGS["long_dna"]
    batch, L, Dn = cfg.batch, cfg.seqlen, cfg.d_inner
    plan = ssm.ssm_scan_bwd_plan_query(batch, L, Dn)
    say(f"backward, long_dna batch {batch} seqlen {L} d_inner {Dn}, planner's plan {plan}")
    assert plan["n_chunks"] > 1
    gen = torch.Generator(device="cuda").manual_seed(41)

    def bf16(shape, scale=1.0, shift=0.0, uniform=False):
        out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        flat = out.view(-1)
        for i in range(0, flat.numel(), 1 << 28):
            n = min(1 << 28, flat.numel() - i)
            r = torch.rand(n, generator=gen, device="cuda") if uniform else torch.randn(n, generator=gen, device="cuda")
            flat[i:i + n] = (r * scale + shift).to(torch.bfloat16)
        return out

    sh = (batch, L, Dn)
    x, z = bf16(sh), bf16(sh)
    dl = bf16(sh, 6.907 - 2.302, -6.907, uniform=True)  # softplus^-1 of steps in [1e-3, 0.1]
    dout = bf16(sh).float()                            # fp32 gradients of bf16-exact values
    B, C = bf16((batch, L, 16)), bf16((batch, L, 16))
    A = -(torch.rand((Dn, 16), generator=gen, device="cuda") * 15.0 + 0.5)
    D = torch.rand(Dn, generator=gen, device="cuda") + 0.5
    bias = torch.rand(Dn, generator=gen, device="cuda") * 0.1
    res = ssm.ssm_scan_bwd(x, dl, A, B, C, D, z, bias, softplus=True, dout=dout)
    torch.cuda.synchronize()

    def np_(t):
        return t.float().cpu().numpy()

    sel = [0, 1023, Dn - 1]
    ref = oracle.scan_bwd(np_(x[..., sel]), np_(dl[..., sel]), np_(A[sel]), np_(B), np_(C), np_(D[sel]),
                          np_(z[..., sel]), np_(bias[sel]), softplus=True, dout=np_(dout[..., sel]))
    for k in ("dx", "ddelta", "dz"):
        assert rowinf(np_(res[k][..., sel]), ref[k], 1) <= TOL, k
    assert rowinf(np_(res["dA"][sel]), ref["dA"], 1) <= TOL
    for k in ("dD", "ddelta_bias"):
        got = np_(res[k][sel])
        assert float(np.max(np.abs(got - ref[k])) / np.max(np.abs(ref[k]))) <= TOL, k
    m = 64
    tail = oracle.scan_bwd(np_(x[:, -m:]), np_(dl[:, -m:]), np_(A), np_(B[:, -m:]), np_(C[:, -m:]), np_(D),
                           np_(z[:, -m:]), np_(bias), softplus=True, dout=np_(dout[:, -m:]))
    assert rowinf(np_(res["dB"][:, -m:]), tail["dB"], 1) <= TOL
    head = oracle.scan_bwd(np_(x[:, :m]), np_(dl[:, :m]), np_(A), np_(B[:, :m]), np_(C[:, :m]), np_(D),
                           np_(z[:, :m]), np_(bias), softplus=True, dout=np_(dout[:, :m]))
    assert rowinf(np_(res["dC"][:, :m]), head["dC"], 1) <= TOL


def test_workspace_pool_keeps_memory_until_trimmed():
    """Workspaces come from the library's own pool, whose freed memory stays mapped
    across synchronisations (so a call after a sync does not map it again) until
    ssm_trim_workspace returns it; results are the same whichever memory a call gets."""
    say("workspace pool: reuse after synchronisation, then trim")
    batch, L, Dn = 2, 4096, 512
    inp, g, gl, h0 = _case(batch, L, Dn, dtype="bf16", seed=21)
    # the checkpoints alone: batch x blocks x tiles x 64 x 16 fp32
    ckpt_bytes = batch * (Dn // 64) * (L // 8) * 64 * 16 * 4
    first = _run(inp, g, gl, h0)
    free1, _ = torch.cuda.mem_get_info()
    second = _run(inp, g, gl, h0)
    free2, _ = torch.cuda.mem_get_info()
    ssm.ssm_trim_workspace()
    torch.cuda.synchronize()
    free3, _ = torch.cuda.mem_get_info()
    third = _run(inp, g, gl, h0)
    for k in first:
        assert np.array_equal(first[k], second[k]) and np.array_equal(first[k], third[k]), k
    say(f"free after call 1 {free1 / 2**20:.0f} MiB, after call 2 {free2 / 2**20:.0f}, after trim {free3 / 2**20:.0f}; "
        f"checkpoints {ckpt_bytes / 2**20:.0f} MiB")
    assert free2 >= free1 - ckpt_bytes // 4, "the second call mapped its workspace again"
    assert free3 - free2 >= ckpt_bytes // 2, "trimming did not return the workspace"


@pytest.mark.parametrize("Dn", [70, 128])
@pytest.mark.parametrize("L,chunk_len", [(203, None), (256, None), (203, 24), (300, 64)])
def test_bwd_structured_A(Dn, L, chunk_len):
    """A with rows (n + 1) A[d, 0]: the forward's checkpoint pass then forms the
    transitions as powers of one exponential; ragged lengths put checkpoints inside
    the forward's peeled first tile, and time chunks start it from carried states."""
    say(f"backward, A rows (n + 1) A[d, 0]: batch 2, L {L}, d_inner {Dn}, chunk_len {chunk_len}")
    inp, g, gl, h0 = _case(2, L, Dn, seed=17)
    a0 = -np.exp(np.random.default_rng(170).uniform(-1.0, 1.5, Dn)).astype(np.float32)
    inp["A"] = (np.arange(1, 17, dtype=np.float32)[None, :] * a0[:, None]).astype(np.float32)
    got = _run(inp, g, gl, h0, chunk_len=chunk_len)
    _compare(got, _ref(inp, g, gl, h0))


@pytest.mark.parametrize("batch,L,Dn,dtype,a_kind", [(2, 37, 70, "f32", "random"), (2, 300, 128, "bf16", "random"),
                                                     (1, 3000, 64, "bf16", "structured"),
                                                     (2, 203, 65, "f32", "structured")])
def test_checkpoints_from_the_forward(batch, L, Dn, dtype, a_kind):
    """ssm_scan_fwd_ckpt keeps the backward's checkpoints while it scans: its out and
    last_state equal ssm_scan_fwd_from's bit for bit.  ssm_scan_bwd_ckpt from them equals
    ssm_scan_bwd bit for bit where neither planner cuts the sequence (the checkpoints are
    then the same states); the 3000-step case is cut, at different points by the two
    planners, so its checkpoints differ by rounding and its gradients are held to the
    oracle instead."""
    say(f"checkpoints from the forward: batch {batch}, L {L}, d_inner {Dn}, {dtype}, A {a_kind}")
    inp, g, gl, h0 = _case(batch, L, Dn, dtype=dtype, seed=31)
    if a_kind == "structured":
        a0 = -np.exp(np.random.default_rng(310).uniform(-1.0, 1.5, Dn)).astype(np.float32)
        inp["A"] = (np.arange(1, 17, dtype=np.float32)[None, :] * a0[:, None]).astype(np.float32)
    t = to_dev(inp)
    h0t = torch.from_numpy(h0).cuda()
    last1 = torch.empty((batch, Dn, 16), device="cuda")
    last2 = torch.empty((batch, Dn, 16), device="cuda")
    out1 = ssm.ssm_scan_fwd_from(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                                 initial_state=h0t, last_state=last1, out_dtype=torch.float32)
    out2, ck = ssm.ssm_scan_fwd_ckpt(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                                     initial_state=h0t, last_state=last2, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(last1, last2)
    dout = torch.from_numpy(g).cuda()   # fp32 gradients, held to the oracle's bar where compared with it
    dlast = torch.from_numpy(gl).cuda()
    kw = dict(softplus=True, initial_state=h0t, dout=dout, dlast_state=dlast, want_dinitial_state=True)
    ref = ssm.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], **kw)
    got = ssm.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], ckpt=ck,
                           **kw)
    torch.cuda.synchronize()
    cut = (ssm.ssm_scan_plan(batch, L, Dn)["n_chunks"] > 1 or ssm.ssm_scan_bwd_plan_query(batch, L, Dn)["n_chunks"] > 1)
    if not cut:
        for k in ref:
            assert torch.equal(ref[k], got[k]), k
    else:
        _compare({k: v.float().cpu().numpy() for k, v in got.items()}, _ref(inp, g, gl, h0))
