"""GPU parity of the causal depthwise conv1d front-end (ssm_conv1d_fwd,
ssm_conv1d_update) against the fp64 oracle, through the C ABI.

Bars: the inputs are identical on both sides (bf16 values are exact in fp32),
so only fp32 rounding separates them: max per-row relative error <= 1e-5
(rows = (b, d) over t) for fp32 out, and bf16 out equals round-to-nearest-even
of fp32 out bitwise.  Caches hold raw inputs and must match exactly.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import rne_bf16_of, rowinf, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ssm = pytest.importorskip("sequence_scan_amd")

TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ssm.library()


def _tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _dev(inp):
    t = {}
    for k, v in inp.items():
        if k == "dtype":
            continue
        x = torch.from_numpy(np.ascontiguousarray(v))
        if k in ("x", "conv_state"):
            x = x.to(_tdt(inp["dtype"]))
        t[k] = x.cuda()
    return t


def _run(inp, silu=True, with_state=True, state_out=True, out_dtype=torch.float32, in_place=False):
    t = _dev(inp)
    batch, L, Dn = inp["x"].shape
    K = inp["weight"].shape[1]
    sin = t.get("conv_state") if with_state else None
    if in_place:
        sout = sin
    elif state_out:
        sout = torch.full((batch, Dn, K), 7.0, dtype=_tdt(inp["dtype"]), device="cuda")
    else:
        sout = None
    out = ssm.ssm_conv1d_fwd(t["x"], t["weight"], t["bias"], silu=silu, conv_state_in=sin, conv_state_out=sout,
                             out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), (sout.float().cpu().numpy() if sout is not None else None)


def _ref(inp, silu=True, with_state=True):
    return oracle.conv1d_fwd(inp["x"], inp["weight"], inp["bias"], silu=silu,
                             conv_state=inp.get("conv_state") if with_state else None)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("Dn", [256, 72, 13])
def test_conv1d_vs_oracle(dtype, K, Dn):
    say(f"conv1d {dtype} K={K} d_inner={Dn}")
    inp = workloads.conv_inputs(2, 97, Dn, K, dtype, seed=K + Dn, with_state=True)
    out, st = _run(inp)
    ref, ref_st = _ref(inp)
    assert rowinf(out, ref, 1) <= TOL
    np.testing.assert_array_equal(st, ref_st)


@pytest.mark.parametrize("silu", [True, False])
def test_conv1d_options(silu):
    say(f"conv1d options silu={silu}, no cache, no bias")
    inp = workloads.conv_inputs(3, 70, 128, 4, "bf16", seed=3)
    inp["bias"] = np.zeros_like(inp["bias"])
    out, _ = _run(inp, silu=silu, with_state=False, state_out=False)
    ref, _ = _ref(inp, silu=silu, with_state=False)
    assert rowinf(out, ref, 1) <= TOL


def test_conv1d_out_dtypes():
    say("conv1d bf16 out equals RNE of fp32 out")
    inp = workloads.conv_inputs(2, 65, 512, 4, "bf16", seed=11, with_state=True)
    o32, _ = _run(inp)
    t = _dev(inp)
    o16 = ssm.ssm_conv1d_fwd(t["x"], t["weight"], t["bias"], conv_state_in=t["conv_state"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o16.float().cpu().numpy(), rne_bf16_of(torch.from_numpy(o32)))


def test_conv1d_short_and_empty_sequences():
    for L in (0, 1, 2, 3, 5):
        say(f"conv1d seqlen {L}")
        inp = workloads.conv_inputs(2, L, 64, 4, "bf16", seed=L, with_state=True)
        out, st = _run(inp)
        ref, ref_st = _ref(inp)
        assert rowinf(out, ref, 1) <= TOL
        np.testing.assert_array_equal(st, ref_st)
        out, st = _run(inp, with_state=False)
        ref, ref_st = _ref(inp, with_state=False)
        np.testing.assert_array_equal(st, ref_st)


@pytest.mark.parametrize("dtype,K,Dn", [("bf16", 4, 200), ("f32", 3, 13), ("bf16", 2, 24), ("f32", 4, 64)])
def test_conv1d_in_place_cache_and_decode(dtype, K, Dn):
    say(f"conv1d {dtype} K={K} d_inner={Dn}: prefill with an in-place cache, then 6 decode steps")
    batch = 3
    inp = workloads.conv_inputs(batch, 45, Dn, K, dtype, seed=21, with_state=True)
    more = workloads.conv_inputs(batch, 6, Dn, K, dtype, seed=22)
    t = _dev(inp)
    cache = t["conv_state"].clone()
    out = ssm.ssm_conv1d_fwd(t["x"], t["weight"], t["bias"], conv_state_in=cache, conv_state_out=cache,
                             out_dtype=torch.float32)
    ref, ref_st = _ref(inp)
    torch.cuda.synchronize()
    assert rowinf(out.cpu().numpy(), ref, 1) <= TOL
    np.testing.assert_array_equal(cache.float().cpu().numpy(), ref_st)
    xs = torch.from_numpy(more["x"]).to(_tdt(dtype)).cuda()
    ys = []
    for s in range(6):
        ys.append(ssm.ssm_conv1d_update(cache, xs[:, s].contiguous(), t["weight"], t["bias"], out_dtype=torch.float32))
    torch.cuda.synchronize()
    got = torch.stack(ys, dim=1).cpu().numpy()
    ref2, ref2_st = oracle.conv1d_fwd(more["x"], inp["weight"], inp["bias"], conv_state=ref_st)
    assert rowinf(got, ref2, 1) <= TOL
    np.testing.assert_array_equal(cache.float().cpu().numpy(), ref2_st)


def test_conv1d_full_size_sampled():
    say("conv1d Mamba-2.8B-like layer: batch 8, seqlen 2048, d_inner 5120, sampled channels")
    inp = workloads.conv_inputs(8, 2048, 5120, 4, "bf16", seed=0, with_state=True)
    out, st = _run(inp)
    sel = np.array(sorted({0, 7, 8, 511, 512, 2049, 4095, 5119, 1234, 3333}))
    sub = dict(inp)
    sub["x"] = np.ascontiguousarray(inp["x"][..., sel])
    sub["weight"] = np.ascontiguousarray(inp["weight"][sel])
    sub["bias"] = np.ascontiguousarray(inp["bias"][sel])
    sub["conv_state"] = np.ascontiguousarray(inp["conv_state"][:, sel])
    ref, ref_st = _ref(sub)
    assert rowinf(out[..., sel], ref, 1) <= TOL
    np.testing.assert_array_equal(st[:, sel], ref_st)
