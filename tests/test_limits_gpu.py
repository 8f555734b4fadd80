"""GPU parity at the limits of the C ABI: the largest batch (65535, one grid
dimension), the largest number of time chunks (65535, another), and tensors of
more than 2^31 elements, whose offsets need 64-bit arithmetic.  Inputs are drawn on the GPU from a seeded generator (the sizes are
too large to draw on the host); the oracle runs on the channels and rows
sampled from the same values."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import rowinf, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ssm = pytest.importorskip("sequence_scan_amd")

TOL_BF16 = 2e-3
N = 16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ssm.library()


def _normal_bf16(shape, gen):
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    flat = out.view(-1)
    step = 1 << 28  # draw in pieces to bound the fp32 temporary
    for i in range(0, flat.numel(), step):
        n = min(step, flat.numel() - i)
        flat[i:i + n] = torch.randn(n, generator=gen, device="cuda").to(torch.bfloat16)
    return out


def _delta_bf16(shape, gen):
    # softplus^-1 of steps log-uniform in [1e-3, 0.1] lies in [-6.907, -2.252]
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    flat = out.view(-1)
    step = 1 << 28
    for i in range(0, flat.numel(), step):
        n = min(step, flat.numel() - i)
        flat[i:i + n] = (torch.rand(n, generator=gen, device="cuda") * 4.655 - 6.907).to(torch.bfloat16)
    return out


def _params(d_inner):
    A = (-torch.arange(1, N + 1, dtype=torch.float32)).repeat(d_inner, 1).contiguous()
    return A.cuda(), torch.ones(d_inner, device="cuda"), torch.zeros(d_inner, device="cuda")


def _np(t):
    return t.float().cpu().numpy()


def test_max_batch_scan_and_decode():
    batch, L, Dn = 65535, 3, 8
    say(f"limits: batch {batch} (the maximum), seqlen {L}, d_inner {Dn}: scan, then one decode step")
    gen = torch.Generator(device="cuda").manual_seed(31)
    x, z = _normal_bf16((batch, L, Dn), gen), _normal_bf16((batch, L, Dn), gen)
    dl = _delta_bf16((batch, L, Dn), gen)
    B, C = _normal_bf16((batch, L, N), gen), _normal_bf16((batch, L, N), gen)
    A, D, bias = _params(Dn)
    last = torch.empty((batch, Dn, N), device="cuda")
    out = ssm.ssm_scan_fwd(x, dl, A, B, C, D, z, bias, out_dtype=torch.float32, last_state=last)
    # one more step from the final state
    xs, ds, zs = x[:, 0].contiguous(), dl[:, 0].contiguous(), z[:, 0].contiguous()
    Bs, Cs = B[:, 0].contiguous(), C[:, 0].contiguous()
    st = last.clone()
    yd = ssm.ssm_state_update(st, xs, ds, A, Bs, Cs, D, zs, bias, out_dtype=torch.float32)
    torch.cuda.synchronize()
    An, Dnp, bn = _np(A), _np(D), _np(bias)
    ref, ref_last = oracle.scan_fwd(_np(x), _np(dl), An, _np(B), _np(C), Dnp, _np(z), bn)
    assert rowinf(_np(out), ref, 1) <= TOL_BF16
    assert rowinf(_np(last), ref_last, 2) <= TOL_BF16
    ref_y, ref_st = oracle.state_update(ref_last, _np(xs), _np(ds), An, _np(Bs), _np(Cs), Dnp, _np(zs), bn)
    assert rowinf(_np(yd), ref_y, 1) <= TOL_BF16  # one step: rows are batch items over channels
    assert rowinf(_np(st), ref_st, 2) <= TOL_BF16


def test_scan_over_2g_elements_sampled():
    batch, L, Dn = 1, (1 << 19) + 5, 4160  # 2.18e9 elements; 65 channel blocks; a ragged tail
    plan = ssm.ssm_scan_plan(batch, L, Dn)
    say(f"limits: scan over {batch * L * Dn / 1e9:.2f}e9 elements (batch {batch}, seqlen {L}, d_inner {Dn}), "
        f"plan {plan}")
    assert batch * L * Dn > 2 ** 31
    gen = torch.Generator(device="cuda").manual_seed(32)
    x, z = _normal_bf16((batch, L, Dn), gen), _normal_bf16((batch, L, Dn), gen)
    dl = _delta_bf16((batch, L, Dn), gen)
    B, C = _normal_bf16((batch, L, N), gen), _normal_bf16((batch, L, N), gen)
    A, D, bias = _params(Dn)
    last = torch.empty((batch, Dn, N), device="cuda")
    out = ssm.ssm_scan_fwd(x, dl, A, B, C, D, z, bias, out_dtype=torch.float32, last_state=last)
    torch.cuda.synchronize()
    sel = [0, 2111, Dn - 1]  # first block, a middle one, the last channel
    ref, ref_last = oracle.scan_fwd(_np(x[:, :, sel]), _np(dl[:, :, sel]), _np(A[sel]), _np(B), _np(C),
                                    _np(D[sel]), _np(z[:, :, sel]), _np(bias[sel]))
    got = _np(out[:, :, sel])
    assert np.all(np.isfinite(got))
    assert rowinf(got, ref, 1) <= TOL_BF16
    assert rowinf(_np(last[:, sel]), ref_last, 2) <= TOL_BF16
    # the last steps of the last channel, where a 32-bit offset would first wrap
    assert rowinf(got[:, -4096:, -1:], ref[:, -4096:, -1:], 1) <= TOL_BF16


def test_decode_over_2g_state_values_sampled():
    batch, Dn = 65535, 2112  # state: 2.21e9 fp32 values
    say(f"limits: decode step with a {batch * Dn * N / 1e9:.2f}e9-value state (batch {batch}, d_inner {Dn})")
    assert batch * Dn * N > 2 ** 31
    gen = torch.Generator(device="cuda").manual_seed(33)
    st = torch.empty((batch, Dn, N), device="cuda")
    flat = st.view(-1)
    for i in range(0, flat.numel(), 1 << 28):
        n = min(1 << 28, flat.numel() - i)
        flat[i:i + n] = torch.randn(n, generator=gen, device="cuda")
    x, z = _normal_bf16((batch, Dn), gen), _normal_bf16((batch, Dn), gen)
    dl = _delta_bf16((batch, Dn), gen)
    B, C = _normal_bf16((batch, N), gen), _normal_bf16((batch, N), gen)
    A, D, bias = _params(Dn)
    rows = [0, 1, 40000, batch - 1]
    st0 = _np(st[rows])
    y = ssm.ssm_state_update(st, x, dl, A, B, C, D, z, bias, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_y, ref_st = oracle.state_update(st0, _np(x[rows]), _np(dl[rows]), _np(A), _np(B[rows]), _np(C[rows]),
                                        _np(D), _np(z[rows]), _np(bias))
    assert rowinf(_np(y[rows]), ref_y, 1) <= TOL_BF16  # one step: rows are batch items over channels
    assert rowinf(_np(st[rows]), ref_st, 2) <= TOL_BF16


def test_conv1d_over_2g_elements_sampled():
    batch, L, Dn, K = 1, (1 << 19) + 5, 4160, 4  # 2.18e9 elements
    say(f"limits: conv1d over {batch * L * Dn / 1e9:.2f}e9 elements (batch {batch}, seqlen {L}, d_inner {Dn})")
    assert batch * L * Dn > 2 ** 31
    gen = torch.Generator(device="cuda").manual_seed(34)
    x = _normal_bf16((batch, L, Dn), gen)
    cache_in = _normal_bf16((batch, Dn, K), gen)
    w = torch.randn((Dn, K), generator=gen, device="cuda") * 0.5
    b = torch.randn((Dn,), generator=gen, device="cuda") * 0.1
    cache_out = torch.empty_like(cache_in)
    out = ssm.ssm_conv1d_fwd(x, w, b, conv_state_in=cache_in, conv_state_out=cache_out, out_dtype=torch.float32)
    torch.cuda.synchronize()
    sel = [0, 2111, Dn - 1]
    ref, ref_st = oracle.conv1d_fwd(_np(x[:, :, sel]), _np(w[sel]), _np(b[sel]), conv_state=_np(cache_in[:, sel]))
    got = _np(out[:, :, sel])
    assert rowinf(got, ref, 1) <= 1e-5
    np.testing.assert_array_equal(_np(cache_out[:, sel]), ref_st)


def test_ssd_over_2g_elements_sampled():
    batch, L, H, P, N2 = 1, (1 << 19) + 37, 64, 64, 128  # 2.15e9 elements; a ragged last chunk
    say(f"limits: Mamba-2 scan over {batch * L * H * P / 1e9:.2f}e9 elements (batch {batch}, seqlen {L}, "
        f"{H} heads x {P}, d_state {N2})")
    assert batch * L * H * P > 2 ** 31
    gen = torch.Generator(device="cuda").manual_seed(35)
    x, z = _normal_bf16((batch, L, H, P), gen), _normal_bf16((batch, L, H, P), gen)
    dt = _delta_bf16((batch, L, H), gen)
    B, C = _normal_bf16((batch, L, 1, N2), gen), _normal_bf16((batch, L, 1, N2), gen)
    A = -(torch.rand(H, generator=gen, device="cuda") * 2.0 + 0.5)
    D = torch.rand(H * P, generator=gen, device="cuda") + 0.5
    bias = torch.zeros(H, device="cuda")
    last = torch.empty((batch, H, P, N2), device="cuda")
    out = ssm.ssm_ssd_fwd(x, dt, A, B, C, D, z, bias, out=torch.empty((batch, L, H, P), device="cuda"),
                          last_state=last)
    torch.cuda.synchronize()
    psel = [0, 17, P - 1]
    for h in (0, H - 1):
        ref, ref_last = oracle.ssd_fwd(_np(x[:, :, h:h + 1, psel]), _np(dt[:, :, h:h + 1]), _np(A[h:h + 1]),
                                       _np(B), _np(C), _np(D[[h * P + p for p in psel]]),
                                       _np(z[:, :, h:h + 1, psel]), _np(bias[h:h + 1]))
        got = _np(out[:, :, h:h + 1, psel])
        assert rowinf(got.reshape(batch, L, -1), ref.reshape(batch, L, -1), 1) <= TOL_BF16
        assert rowinf(_np(last[:, h:h + 1, psel]).reshape(batch, len(psel), N2),
                      ref_last.reshape(batch, len(psel), N2), 2) <= TOL_BF16


def _host_case(batch, L, Dn, seed):
    cfg = workloads.ScanConfig("limit", batch, Dn, N, L, "bf16")
    inp = workloads.scan_inputs(cfg, seed=seed, random_params=True)
    rng = np.random.default_rng(seed)
    g = workloads.round_to_bf16(rng.standard_normal((batch, L, Dn)).astype(np.float32))
    return inp, g


def _dev(inp):
    return {k: (torch.from_numpy(v).to(torch.bfloat16) if k in ("x", "delta", "z", "B", "C") else torch.from_numpy(v)).cuda()
            for k, v in inp.items() if k != "dtype"}


def _bwd_errs(got, ref, per_item=False):
    """Row-relative errors of the backward's gradients: rows over t as in the
    backward's parity tests, or (per_item) whole batch items, for sequences too
    short for a row over t to have a meaningful scale."""
    errs = {}
    for k in ("dx", "ddelta", "dz", "dB", "dC"):
        gk, rk = got[k].float().cpu().numpy(), ref[k]
        if per_item:
            gk, rk = gk.reshape(gk.shape[0], -1), rk.reshape(rk.shape[0], -1)
        errs[k] = rowinf(gk, rk, 1)
    errs["dA"] = rowinf(got["dA"].float().cpu().numpy(), ref["dA"], 1)
    for k in ("dD", "ddelta_bias"):
        r = ref[k]
        errs[k] = float(np.max(np.abs(got[k].float().cpu().numpy() - r)) / np.max(np.abs(r)))
    return errs


def test_max_chunks_scan_and_backward():
    L, Dn = 65535 * 8, 8   # 8-step chunks: 65535 of them, the largest plan
    say(f"limits: forward and backward in 65535 time chunks of 8 steps (batch 1, seqlen {L}, d_inner {Dn})")
    inp, g = _host_case(1, L, Dn, seed=36)
    t = _dev(inp)
    plan = {"states_per_wave": 4, "chunk_len": 8}
    last = torch.empty((1, Dn, N), device="cuda")
    out = ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                           out_dtype=torch.float32, last_state=last, plan=plan)
    res = ssm.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                           dout=torch.from_numpy(g).cuda(), plan=plan)
    torch.cuda.synchronize()
    ref, ref_last = oracle.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                    inp["delta_bias"])
    assert rowinf(_np(out), ref, 1) <= TOL_BF16
    assert rowinf(_np(last), ref_last, 2) <= TOL_BF16
    refg = oracle.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                           inp["delta_bias"], softplus=True, dout=g)
    for k, e in _bwd_errs(res, refg).items():
        assert e <= 1e-4, f"{k}: {e:.3e}"


def test_max_batch_backward():
    batch, L, Dn = 65535, 3, 8
    say(f"limits: backward at batch {batch} (the maximum), seqlen {L}, d_inner {Dn}")
    inp, g = _host_case(batch, L, Dn, seed=37)
    t = _dev(inp)
    res = ssm.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                           dout=torch.from_numpy(g).cuda())
    torch.cuda.synchronize()
    refg = oracle.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                           inp["delta_bias"], softplus=True, dout=g)
    errs = _bwd_errs(res, refg, per_item=True)  # three steps: rows are batch items
    say("errors: " + " ".join(f"{k}={e:.1e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert e <= 1e-4, f"{k}: {e:.3e}"
