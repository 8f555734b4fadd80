"""C-ABI checks that run without a GPU: exports, versions, status strings, and
every host-side rejection path (these return before any HIP call is made)."""
import ctypes
import os
import re

import pytest

import sequence_scan_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(ssm.HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(ssm_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_function_is_exported():
    lib = ssm.library()
    names = header_functions()
    assert {"ssm_scan_fwd", "ssm_state_update", "ssm_scan_plan", "ssm_scan_fwd_plan", "ssm_scan_fwd_from",
            "ssm_conv1d_fwd", "ssm_conv1d_update", "ssm_affine_exclusive_scan", "ssm_status_string",
            "ssm_last_error", "ssm_abi_version", "ssm_scan_bwd", "ssm_scan_bwd_plan", "ssm_scan_bwd_plan_query",
            "ssm_ssd_fwd", "ssm_ssd_fwd_plan", "ssm_ssd_plan_query", "ssm_ssd_state_update",
            "ssm_scan_fwd_noalloc", "ssm_trim_workspace", "ssm_scan_ckpt_bytes", "ssm_scan_fwd_ckpt",
            "ssm_scan_bwd_ckpt"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ssmscan.h but not exported"


def test_probe_library_exports():
    """The benchmark's probe library (VALU issue rates, streaming bandwidth) is
    separate from the scan library and exports its launchers."""
    from sequence_scan_amd import build as lib_build
    probe = ctypes.CDLL(lib_build.PROBE_LIB)
    for n in ("ssm_probe_launch", "ssm_probe_ops_per_iter", "ssm_stream_probe_launch"):
        assert hasattr(probe, n)
    lib = ssm.library()
    assert not hasattr(lib, "ssm_stream_probe_launch") and not hasattr(lib, "ssm_probe_launch")


def test_version_and_strings():
    assert ssm.ssm_abi_version() == 10
    for code, name in ssm.STATUS_NAMES.items():
        assert ssm.ssm_status_string(code).startswith(name)
    assert "unknown" in ssm.ssm_status_string(99)


F32, BF16 = ssm.SSM_F32, ssm.SSM_BF16
P = 0x10000000  # fake, 16-byte aligned device addresses: never dereferenced on these paths


def scan(**kw):
    a = dict(x=P, delta=P + 0x1000000, A=P + 0x2000000, B=P + 0x3000000, C=P + 0x4000000, D=None, z=None,
             bias=None, softplus=1, out=P + 0x5000000, last=None, batch=2, seqlen=8, d_inner=64, d_state=16,
             ind=F32, outd=F32, stream=None)
    a.update(kw)
    lib = ssm.library()
    return lib.ssm_scan_fwd(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["softplus"],
                            a["out"], a["last"], a["batch"], a["seqlen"], a["d_inner"], a["d_state"], a["ind"],
                            a["outd"], a["stream"])


@pytest.mark.parametrize("arg", ["x", "delta", "A", "B", "C", "out"])
def test_null_required(arg):
    assert scan(**{arg: None}) == ssm.SSM_ERR_NULL_ARG
    assert arg in ssm.ssm_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), ssm.SSM_ERR_BAD_SHAPE),
    (dict(seqlen=-5), ssm.SSM_ERR_BAD_SHAPE),
    (dict(d_inner=-64), ssm.SSM_ERR_BAD_SHAPE),
    (dict(batch=1 << 40, seqlen=1 << 20, d_inner=1 << 10), ssm.SSM_ERR_BAD_SHAPE),
    (dict(d_state=8), ssm.SSM_ERR_UNSUPPORTED),
    (dict(d_state=32), ssm.SSM_ERR_UNSUPPORTED),
    (dict(ind=7), ssm.SSM_ERR_UNSUPPORTED),
    (dict(outd=-1), ssm.SSM_ERR_UNSUPPORTED),
    (dict(batch=70000, seqlen=1, d_inner=1), ssm.SSM_ERR_UNSUPPORTED),
])
def test_bad_sizes_and_types(kw, code):
    assert scan(**kw) == code
    assert ssm.ssm_last_error() != ""


@pytest.mark.parametrize("arg", ["x", "delta", "A", "B", "C", "D", "z", "bias", "out", "last"])
def test_misaligned(arg):
    kw = {"D": P + 0x6000000, "z": P + 0x7000000, "bias": P + 0x8000000, "last": P + 0x9000000}
    base = {**kw}
    cur = {"x": P, "delta": P + 0x1000000, "A": P + 0x2000000, "B": P + 0x3000000, "C": P + 0x4000000,
           "out": P + 0x5000000, **base}
    cur[arg] = cur[arg] + 4
    assert scan(**cur) == ssm.SSM_ERR_UNSUPPORTED
    assert "aligned" in ssm.ssm_last_error()


@pytest.mark.parametrize("target", ["x", "delta", "B", "A"])
def test_out_aliasing_an_input(target):
    ptrs = {"x": P, "delta": P + 0x1000000, "A": P + 0x2000000, "B": P + 0x3000000}
    assert scan(out=ptrs[target] + 16) == ssm.SSM_ERR_UNSUPPORTED
    assert "overlaps" in ssm.ssm_last_error()


def test_last_state_aliasing():
    assert scan(last=P + 0x1000000 + 64) == ssm.SSM_ERR_UNSUPPORTED
    assert scan(last=P + 0x5000000 + 32) == ssm.SSM_ERR_UNSUPPORTED


def test_bad_plan_rejected_before_launch():
    lib = ssm.library()
    for spw, chunk in ((3, 10), (32, 10), (4, 0), (4, -3)):
        p = ssm.ssm_plan()
        p.states_per_wave = spw
        p.chunk_len = chunk
        rc = lib.ssm_scan_fwd_plan(P, P + 0x1000000, P + 0x2000000, P + 0x3000000, P + 0x4000000, None, None, None,
                                   1, P + 0x5000000, None, 2, 8, 64, 16, F32, F32, None, ctypes.byref(p))
        assert rc == ssm.SSM_ERR_UNSUPPORTED, (spw, chunk)
    assert lib.ssm_scan_fwd_plan(P, P, P, P, P, None, None, None, 1, P, None, 1, 1, 1, 16, F32, F32, None,
                                 None) == ssm.SSM_ERR_NULL_ARG


def test_decode_rejections():
    lib = ssm.library()

    def dec(**kw):
        a = dict(state=P, x=P + 0x1000000, delta=P + 0x2000000, A=P + 0x3000000, B=P + 0x4000000, C=P + 0x5000000,
                 D=None, z=None, bias=None, softplus=1, out=P + 0x6000000, batch=4, d_inner=64, d_state=16,
                 ind=BF16, outd=F32)
        a.update(kw)
        return lib.ssm_state_update(a["state"], a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                    a["bias"], a["softplus"], a["out"], a["batch"], a["d_inner"], a["d_state"],
                                    a["ind"], a["outd"], None)
    assert dec(state=None) == ssm.SSM_ERR_NULL_ARG
    assert dec(out=None) == ssm.SSM_ERR_NULL_ARG
    assert dec(batch=-1) == ssm.SSM_ERR_BAD_SHAPE
    assert dec(d_state=4) == ssm.SSM_ERR_UNSUPPORTED
    assert dec(state=P + 8) == ssm.SSM_ERR_UNSUPPORTED
    assert dec(out=P + 32) == ssm.SSM_ERR_UNSUPPORTED          # out inside state
    assert dec(state=P + 0x1000000) == ssm.SSM_ERR_UNSUPPORTED  # state on x


def test_affine_scan_rejections():
    lib = ssm.library()
    assert lib.ssm_affine_exclusive_scan(P, P, P, P, -1, None) == ssm.SSM_ERR_BAD_SHAPE
    assert lib.ssm_affine_exclusive_scan(None, P, P, P, 3, None) == ssm.SSM_ERR_NULL_ARG


def test_plan_choices():
    # Sizes of the benchmark workloads (MI355X: 256 CUs = 1024 SIMDs).
    p = ssm.ssm_scan_plan(8, 2048, 5120)
    assert p["n_chunks"] == 1 and p["states_per_wave"] == 4
    p = ssm.ssm_scan_plan(1, 262144, 2048)
    assert p["n_chunks"] > 1 and p["chunk_len"] * p["n_chunks"] >= 262144
    assert p["chunk_len"] % 32 == 0 and p["chunk_len"] * (p["n_chunks"] - 1) < 262144   # cut at whole tiles
    assert (p["chunk_len"], p["n_chunks"]) == (2752, 96)
    p = ssm.ssm_scan_plan(8, 2048, 1536)   # 192 blocks for 256 CUs: about three workgroups per CU
    assert p["n_chunks"] == 4 and p["chunk_len"] == 512
    p = ssm.ssm_scan_plan(8, 700, 1536)    # too short to cut into chunks of 512
    assert p["n_chunks"] == 1
    p = ssm.ssm_scan_plan(1, 0, 64)
    assert p["n_chunks"] == 0
    with pytest.raises(ssm.SSMError):
        ssm.ssm_scan_plan(1, 10, 64, 12)


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(ssm, "_lib", None)
    monkeypatch.setattr(ssm, "LIB_PATH", os.path.join(ROOT, "does-not-exist.so"))
    with pytest.raises(RuntimeError, match="not built"):
        ssm.library()


def test_product_code_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "sequence_scan_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f"{f} mentions the oracle"
    hdr = open(ssm.HEADER_PATH).read().lower()
    assert "oracle" not in hdr


def test_scan_from_state_rejections():
    lib = ssm.library()

    def run(h0, last, out=P + 0x5000000):
        return lib.ssm_scan_fwd_from(P, P + 0x1000000, P + 0x2000000, P + 0x3000000, P + 0x4000000, None, None, None,
                                     1, h0, out, last, 2, 8, 64, 16, F32, F32, None, None)
    assert run(P + 0x6000000 + 4, None) == ssm.SSM_ERR_UNSUPPORTED           # misaligned initial state
    assert "aligned" in ssm.ssm_last_error()
    assert run(P + 0x6000000, P + 0x6000000 + 16) == ssm.SSM_ERR_UNSUPPORTED  # partial overlap
    assert "initial_state" in ssm.ssm_last_error()
    assert run(P + 0x5000000, None) == ssm.SSM_ERR_UNSUPPORTED                # out over the initial state
    bad = ssm.ssm_plan()
    bad.states_per_wave, bad.chunk_len = 3, 8
    assert lib.ssm_scan_fwd_from(P, P, P, P, P, None, None, None, 1, None, P + 0x5000000, None, 1, 8, 64, 16,
                                 F32, F32, None, ctypes.byref(bad)) == ssm.SSM_ERR_UNSUPPORTED


def test_noalloc_rejections():
    """The entry point that allocates nothing checks what ssm_scan_fwd_from checks, and
    rejects a plan whose carry workspace exceeds its fixed scratch, before any HIP call."""
    lib = ssm.library()
    G = 0x10000000000  # 1 TiB apart: the fake tensors never overlap

    def run(batch, seqlen, d_inner, chunk, x=P, h0=None, last=None):
        pl = ssm.ssm_plan()
        pl.states_per_wave, pl.chunk_len = 4, chunk
        return lib.ssm_scan_fwd_noalloc(x, P + G, P + 2 * G, P + 3 * G, P + 4 * G, None, None, None, 1, h0,
                                        P + 5 * G, last, batch, seqlen, d_inner, 16, BF16, F32, None,
                                        ctypes.byref(pl))
    # batch 8 x 5120 channels in 16 chunks: 8 * 16 * 5120 * 17 * 4 bytes = 44.6 MB > 32 MiB
    assert run(8, 2048, 5120, 128) == ssm.SSM_ERR_UNSUPPORTED
    msg = ssm.ssm_last_error()
    assert "scratch" in msg and str(32 * 1024 * 1024) in msg
    assert run(8, 2048, 5120, 512, h0=P + 6 * G, last=P + 6 * G + 16) == ssm.SSM_ERR_UNSUPPORTED  # partial overlap
    assert "initial_state" in ssm.ssm_last_error()
    assert run(8, 2048, 5120, 128, x=None) == ssm.SSM_ERR_NULL_ARG
    assert run(8, 2048, 5120, 128, x=P + 4) == ssm.SSM_ERR_UNSUPPORTED and "aligned" in ssm.ssm_last_error()
    assert run(0, 2048, 5120, 128) == ssm.SSM_OK          # empty: nothing to do, nothing looked up
    assert lib.ssm_scan_fwd_noalloc(P, P + G, P + 2 * G, P + 3 * G, P + 4 * G, None, None, None, 4, None,
                                    P + 5 * G, None, 1, 8, 64, 16, F32, F32, None, None) == ssm.SSM_ERR_UNSUPPORTED


def test_checkpoint_calls_rejections():
    """The calls that hand the backward's checkpoints from the forward: their size, and
    the host checks of ssm_scan_fwd_ckpt / ssm_scan_bwd_ckpt (nothing is enqueued)."""
    lib = ssm.library()
    G = 0x10000000000  # 1 TiB apart: the fake tensors never overlap
    assert ssm.ssm_scan_ckpt_bytes(8, 2048, 5120) == 8 * 80 * 256 * 1024 * 4
    assert ssm.ssm_scan_ckpt_bytes(2, 37, 70) == 2 * 2 * 5 * 1024 * 4       # ragged tiles and channel blocks
    n = ctypes.c_int64(0)
    assert lib.ssm_scan_ckpt_bytes(8, 2048, 5120, 8, ctypes.byref(n)) == ssm.SSM_ERR_UNSUPPORTED
    assert lib.ssm_scan_ckpt_bytes(8, -1, 5120, 16, ctypes.byref(n)) == ssm.SSM_ERR_BAD_SHAPE
    assert lib.ssm_scan_ckpt_bytes(8, 2048, 5120, 16, None) == ssm.SSM_ERR_NULL_ARG

    def fwd(ckpt, flags=1, out=P + 5 * G):
        return lib.ssm_scan_fwd_ckpt(P, P + G, P + 2 * G, P + 3 * G, P + 4 * G, None, None, None, flags, None, out,
                                     None, ckpt, 8, 2048, 5120, 16, BF16, F32, None)
    assert fwd(None) == ssm.SSM_ERR_NULL_ARG and "ckpt" in ssm.ssm_last_error()
    assert fwd(P + 6 * G, flags=3) == ssm.SSM_ERR_UNSUPPORTED and "ZOH" in ssm.ssm_last_error()
    assert fwd(P + 6 * G + 4) == ssm.SSM_ERR_UNSUPPORTED and "aligned" in ssm.ssm_last_error()
    assert fwd(P + 5 * G + 1024) == ssm.SSM_ERR_UNSUPPORTED and "ckpt" in ssm.ssm_last_error()  # inside out
    assert fwd(P + G) == ssm.SSM_ERR_UNSUPPORTED and "ckpt" in ssm.ssm_last_error()             # on delta

    def bwd(ckpt, dx=P + 7 * G):
        return lib.ssm_scan_bwd_ckpt(P, P + G, P + 2 * G, P + 3 * G, P + 4 * G, None, None, None, 1, None, P + 5 * G,
                                     None, ckpt, dx, P + 8 * G, P + 9 * G, P + 10 * G, P + 11 * G, None, None, None,
                                     None, 8, 2048, 5120, 16, BF16, BF16, None)
    assert bwd(None) == ssm.SSM_ERR_NULL_ARG and "ckpt" in ssm.ssm_last_error()
    assert bwd(P + 6 * G + 8) == ssm.SSM_ERR_UNSUPPORTED and "aligned" in ssm.ssm_last_error()
    assert bwd(P + 6 * G, dx=P + 6 * G + 4096) == ssm.SSM_ERR_UNSUPPORTED and "ckpt" in ssm.ssm_last_error()


def test_failed_workspace_allocation_is_reported():
    """Without a usable device a chunked plan's workspace allocation fails: the call returns
    SSM_ERR_HIP naming the allocation.  (That a later valid call is not handed the same
    error again is checked on the GPU, where the failure is forced by size.)"""
    lib = ssm.library()
    import torch
    if torch.cuda.is_available():
        pytest.skip("needs a host without a GPU (the GPU suite forces the failure by size)")
    pl = ssm.ssm_plan()
    pl.states_per_wave, pl.chunk_len = 4, 4
    st = lib.ssm_scan_fwd_plan(P, P + 0x1000000, P + 0x2000000, P + 0x3000000, P + 0x4000000, None, None, None, 1,
                               P + 0x5000000, None, 2, 8, 64, 16, F32, F32, None, ctypes.byref(pl))
    assert st == ssm.SSM_ERR_HIP and "workspace allocation" in ssm.ssm_last_error()


def test_conv1d_rejections():
    lib = ssm.library()

    def fwd(**kw):
        a = dict(x=P, w=P + 0x1000000, bias=None, silu=1, sin=None, out=P + 0x2000000, sout=None, batch=2, seqlen=8,
                 d_inner=64, d_conv=4, ind=BF16, outd=BF16)
        a.update(kw)
        return lib.ssm_conv1d_fwd(a["x"], a["w"], a["bias"], a["silu"], a["sin"], a["out"], a["sout"], a["batch"],
                                  a["seqlen"], a["d_inner"], a["d_conv"], a["ind"], a["outd"], None)
    assert fwd(x=None) == ssm.SSM_ERR_NULL_ARG
    assert fwd(w=None) == ssm.SSM_ERR_NULL_ARG
    assert fwd(out=None) == ssm.SSM_ERR_NULL_ARG
    assert fwd(seqlen=-1) == ssm.SSM_ERR_BAD_SHAPE
    for k in (0, 1, 5, 8):
        assert fwd(d_conv=k) == ssm.SSM_ERR_UNSUPPORTED, k
    assert fwd(ind=5) == ssm.SSM_ERR_UNSUPPORTED
    assert fwd(out=P + 8) == ssm.SSM_ERR_UNSUPPORTED                        # misaligned and on x
    assert fwd(out=P + 0x40) == ssm.SSM_ERR_UNSUPPORTED                      # out overlaps x
    assert "overlaps" in ssm.ssm_last_error()
    assert fwd(sin=P + 0x3000000, sout=P + 0x3000000 + 16) == ssm.SSM_ERR_UNSUPPORTED  # partial cache overlap
    assert fwd(sout=P + 0x2000000) == ssm.SSM_ERR_UNSUPPORTED               # cache over out

    def upd(**kw):
        a = dict(st=P, x=P + 0x1000000, w=P + 0x2000000, bias=None, silu=1, out=P + 0x3000000, batch=4, d_inner=64,
                 d_conv=4, ind=BF16, outd=F32)
        a.update(kw)
        return lib.ssm_conv1d_update(a["st"], a["x"], a["w"], a["bias"], a["silu"], a["out"], a["batch"],
                                     a["d_inner"], a["d_conv"], a["ind"], a["outd"], None)
    assert upd(st=None) == ssm.SSM_ERR_NULL_ARG
    assert upd(d_conv=6) == ssm.SSM_ERR_UNSUPPORTED
    assert upd(out=P + 16) == ssm.SSM_ERR_UNSUPPORTED                       # out inside the cache
    assert upd(st=P + 0x1000000) == ssm.SSM_ERR_UNSUPPORTED                 # cache on x


def test_scan_bwd_rejections():
    lib = ssm.library()
    base = dict(x=P, delta=P + 0x1000000, A=P + 0x2000000, B=P + 0x3000000, C=P + 0x4000000, D=None, z=None, bias=None,
                h0=None, dout=P + 0x5000000, dlast=None, dx=P + 0x6000000, ddelta=P + 0x7000000, dA=P + 0x8000000,
                dB=P + 0x9000000, dC=P + 0xa000000, dD=None, dz=None, dbias=None, dh0=None, batch=2, seqlen=8,
                d_inner=64, d_state=16, ind=F32, gd=F32, flags=1)

    def bwd(**kw):
        a = dict(base)
        a.update(kw)
        return lib.ssm_scan_bwd(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["flags"],
                                a["h0"],
                                a["dout"], a["dlast"], a["dx"], a["ddelta"], a["dA"], a["dB"], a["dC"], a["dD"],
                                a["dz"], a["dbias"], a["dh0"], a["batch"], a["seqlen"], a["d_inner"], a["d_state"],
                                a["ind"], a["gd"], None)
    for k in ("dout", "dx", "ddelta", "dA", "dB", "dC"):
        assert bwd(**{k: None}) == ssm.SSM_ERR_NULL_ARG, k
    assert bwd(D=P + 0xb000000) == ssm.SSM_ERR_NULL_ARG                     # D given, dD missing
    assert bwd(dz=P + 0xb000000) == ssm.SSM_ERR_UNSUPPORTED                 # dz without z
    assert bwd(d_state=8) == ssm.SSM_ERR_UNSUPPORTED
    assert bwd(dx=P + 0x6000000 + 4) == ssm.SSM_ERR_UNSUPPORTED             # misaligned
    assert bwd(dx=P + 0x1000000) == ssm.SSM_ERR_UNSUPPORTED                 # dx over delta
    assert bwd(dB=P + 0x6000000 + 64) == ssm.SSM_ERR_UNSUPPORTED            # two gradients overlap
    assert "overlaps" in ssm.ssm_last_error()
    for flags in (ssm.SSM_ZOH, ssm.SSM_ZOH | ssm.SSM_SOFTPLUS):             # the backward of ZOH is not defined
        assert bwd(flags=flags) == ssm.SSM_ERR_UNSUPPORTED
        assert "SSM_ZOH" in ssm.ssm_last_error()
    assert bwd(flags=4) == ssm.SSM_ERR_UNSUPPORTED


def test_bwd_plan_choices():
    # MI355X: 256 CUs.  The layer has 640 blocks: one chunk.
    p = ssm.ssm_scan_bwd_plan_query(8, 2048, 5120)
    assert p["n_chunks"] == 1 and p["states_per_wave"] == 4
    p = ssm.ssm_scan_bwd_plan_query(8, 2048, 1536)    # 192 blocks: chunks of the 512-step minimum
    assert p["n_chunks"] == 4 and p["chunk_len"] == 512
    p = ssm.ssm_scan_bwd_plan_query(7, 2048, 4096)    # 448 blocks = 1.75 per CU: still cut
    assert p["n_chunks"] == 4
    p = ssm.ssm_scan_bwd_plan_query(8, 2048, 4096)    # 512 blocks: one chunk
    assert p["n_chunks"] == 1
    p = ssm.ssm_scan_bwd_plan_query(1, 262144, 2048)  # 32 blocks: about 24 workgroups per CU
    assert p["n_chunks"] == 192 and p["chunk_len"] % 8 == 0 and p["chunk_len"] * p["n_chunks"] >= 262144
    assert p["chunk_len"] * (p["n_chunks"] - 1) < 262144
    p = ssm.ssm_scan_bwd_plan_query(2, 300, 200)      # too short to cut
    assert p["n_chunks"] == 1
    p = ssm.ssm_scan_bwd_plan_query(1, 0, 64)
    assert p["n_chunks"] == 0
    with pytest.raises(ssm.SSMError):
        ssm.ssm_scan_bwd_plan_query(1, 10, 64, 12)


def test_bwd_bad_plan_rejected_before_launch():
    lib = ssm.library()

    def bwd(spw, chunk, seqlen=100, plan=True):
        p = ssm.ssm_plan()
        p.states_per_wave = spw
        p.chunk_len = chunk
        return lib.ssm_scan_bwd_plan(P, P + 0x1000000, P + 0x2000000, P + 0x3000000, P + 0x4000000, None, None, None, 1,
                                     None, P + 0x5000000, None, P + 0x6000000, P + 0x7000000, P + 0x8000000,
                                     P + 0x9000000, P + 0xa000000, None, None, None, None, 1, seqlen, 64, 16, F32, F32,
                                     None, ctypes.byref(p) if plan else None)
    for spw, chunk, seqlen in ((2, 16, 100), (8, 16, 100), (4, 0, 100), (4, -8, 100),
                               (4, 12, 100),       # cuts the sequence at a step that is not a tile boundary
                               (4, 8, 600000)):    # more than 65535 chunks
        assert bwd(spw, chunk, seqlen) == ssm.SSM_ERR_UNSUPPORTED, (spw, chunk, seqlen)
    assert "multiple of 8" in (bwd(4, 12) and ssm.ssm_last_error())
    assert bwd(4, 16, plan=False) == ssm.SSM_ERR_NULL_ARG


def test_step_flags():
    """SSM_SOFTPLUS and SSM_ZOH are the only bits of the step-flags word; valid
    words pass the checks (shown on empty calls, which enqueue nothing)."""
    lib = ssm.library()
    for bad in (4, 8, -1, 1 << 20, 7):
        assert scan(softplus=bad) == ssm.SSM_ERR_UNSUPPORTED, bad
        assert "flags" in ssm.ssm_last_error()
        assert lib.ssm_state_update(P, P + 0x1000000, P + 0x2000000, P + 0x3000000, P + 0x4000000, P + 0x5000000,
                                    None, None, None, bad, P + 0x6000000, 4, 64, 16, F32, F32,
                                    None) == ssm.SSM_ERR_UNSUPPORTED
    for good in (0, ssm.SSM_SOFTPLUS, ssm.SSM_ZOH, ssm.SSM_SOFTPLUS | ssm.SSM_ZOH):
        assert scan(softplus=good, batch=0) == ssm.SSM_OK, good
        assert lib.ssm_state_update(P, P + 0x1000000, P + 0x2000000, P + 0x3000000, P + 0x4000000, P + 0x5000000,
                                    None, None, None, good, P + 0x6000000, 0, 64, 16, F32, F32, None) == ssm.SSM_OK


def test_ssd_plan_choices_and_rejections():
    # MI355X: 256 CUs.  The Mamba-2-2.7B-like layer (640 workgroups) runs in one chunk; one long row is cut.
    p = ssm.ssm_ssd_plan_query(8, 2048, 80, 64, 1, 128)
    assert p["n_chunks"] == 1
    p = ssm.ssm_ssd_plan_query(1, 262144, 32, 64, 1, 128)
    assert p["n_chunks"] > 1 and p["chunk_len"] % 32 == 0 and p["chunk_len"] >= 1024
    assert p["chunk_len"] * p["n_chunks"] >= 262144 > p["chunk_len"] * (p["n_chunks"] - 1)
    assert ssm.ssm_ssd_plan_query(1, 1000, 2, 64, 1, 128)["n_chunks"] == 1     # too short to cut
    with pytest.raises(ssm.SSMError):
        ssm.ssm_ssd_plan_query(1, 10, 4, 32, 1, 128)                            # headdim 32
    lib = ssm.library()

    def ssd(chunk, seqlen=100, plan=True):
        pl = ssm.ssm_plan()
        pl.chunk_len = chunk
        return lib.ssm_ssd_fwd_plan(P, P + 0x1000000, P + 0x2000000, P + 0x3000000, P + 0x4000000, None, None, None, 1,
                                    None, P + 0x5000000, None, 1, seqlen, 4, 64, 1, 128, BF16, F32, None,
                                    ctypes.byref(pl) if plan else None)
    for chunk, seqlen in ((0, 100), (-32, 100), (48, 100), (32, 65536 * 32)):
        assert ssd(chunk, seqlen) == ssm.SSM_ERR_UNSUPPORTED, (chunk, seqlen)
    assert "multiple of 32" in (ssd(48) and ssm.ssm_last_error())
    assert ssd(32, plan=False) == ssm.SSM_ERR_NULL_ARG

    def ssd_heads(nheads, chunk, seqlen=64):
        pl = ssm.ssm_plan()
        pl.chunk_len = chunk
        return lib.ssm_ssd_fwd_plan(P, P + 0x10000000000, P + 0x20000000000, P + 0x30000000000, P + 0x40000000000,
                                    None, None, None, 1, None, P + 0x50000000000, None, 1, seqlen, nheads, 64, 1, 128,
                                    BF16, F32, None, ctypes.byref(pl))
    # at most 65535 heads, chunked (the carry's grid axis) or not (the kernel's
    # 32-bit offsets within a chunk)
    assert ssd_heads(65536, 32) == ssm.SSM_ERR_UNSUPPORTED and "65535" in ssm.ssm_last_error()
    assert ssd_heads(65536, 64) == ssm.SSM_ERR_UNSUPPORTED and "65535" in ssm.ssm_last_error()


def test_ssd_rejections():
    """Host-side checks of the Mamba-2 calls (nothing is enqueued on these paths)."""
    lib = ssm.library()

    def ssd(**kw):
        a = dict(x=P, dt=P + 0x1000000, A=P + 0x2000000, B=P + 0x3000000, C=P + 0x4000000, D=None, z=None, bias=None,
                 flags=1, h0=None, out=P + 0x5000000, last=None, batch=2, seqlen=8, nheads=4, headdim=64, ngroups=2,
                 d_state=128, ind=BF16, outd=F32)
        a.update(kw)
        return lib.ssm_ssd_fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["flags"], a["h0"],
                               a["out"], a["last"], a["batch"], a["seqlen"], a["nheads"], a["headdim"], a["ngroups"],
                               a["d_state"], a["ind"], a["outd"], None)
    for k in ("x", "dt", "A", "B", "C", "out"):
        assert ssd(**{k: None}) == ssm.SSM_ERR_NULL_ARG, k
    assert ssd(ind=F32) == ssm.SSM_ERR_UNSUPPORTED and "bf16" in ssm.ssm_last_error()
    assert ssd(headdim=32) == ssm.SSM_ERR_UNSUPPORTED
    assert ssd(d_state=16) == ssm.SSM_ERR_UNSUPPORTED
    assert ssd(ngroups=3) == ssm.SSM_ERR_UNSUPPORTED                         # 4 heads in 3 groups
    assert ssd(ngroups=0) == ssm.SSM_ERR_UNSUPPORTED
    assert ssd(flags=ssm.SSM_ZOH) == ssm.SSM_ERR_UNSUPPORTED
    assert ssd(seqlen=-1) == ssm.SSM_ERR_BAD_SHAPE
    assert ssd(x=P + 8) == ssm.SSM_ERR_UNSUPPORTED and "aligned" in ssm.ssm_last_error()
    assert ssd(dt=P + 0x1000000 + 1) == ssm.SSM_ERR_UNSUPPORTED               # dt: element alignment
    assert ssd(dt=P + 0x1000000 + 2, batch=0) == ssm.SSM_OK
    assert ssd(out=P + 0x1000000) == ssm.SSM_ERR_UNSUPPORTED                 # out on dt
    assert ssd(last=P + 0x6000000, h0=P + 0x6000000 + 256) == ssm.SSM_ERR_UNSUPPORTED  # partial overlap
    assert ssd(last=P + 0x6000000, h0=P + 0x6000000, batch=0) == ssm.SSM_OK     # in place is allowed
    assert ssd(batch=0) == ssm.SSM_OK

    def upd(**kw):
        a = dict(state=P, x=P + 0x1000000, dt=P + 0x2000000, A=P + 0x3000000, B=P + 0x4000000, C=P + 0x5000000,
                 out=P + 0x6000000, batch=2, nheads=4, headdim=48, ngroups=1, d_state=64, ind=F32)
        a.update(kw)
        return lib.ssm_ssd_state_update(a["state"], a["x"], a["dt"], a["A"], a["B"], a["C"], None, None, None, 1,
                                        a["out"], a["batch"], a["nheads"], a["headdim"], a["ngroups"], a["d_state"],
                                        a["ind"], F32, None)
    assert upd(state=None) == ssm.SSM_ERR_NULL_ARG
    assert upd(d_state=32) == ssm.SSM_ERR_UNSUPPORTED
    assert upd(out=P + 64) == ssm.SSM_ERR_UNSUPPORTED                        # out inside the state
    assert upd(nheads=65536, ngroups=1) == ssm.SSM_ERR_UNSUPPORTED and "65535" in ssm.ssm_last_error()
    assert upd(batch=0) == ssm.SSM_OK


def test_binding_checks_tensor_shapes_and_dtypes():
    """The binding checks every tensor against the sizes it passes to the C ABI (which
    trusts them) before anything is launched; CPU tensors reach the device check last."""
    torch = pytest.importorskip("torch")
    f32, bf = torch.float32, torch.bfloat16
    x, A, B = torch.zeros(2, 5, 8), torch.zeros(8, 16), torch.zeros(2, 5, 16)
    with pytest.raises(ValueError, match="delta"):
        ssm.ssm_scan_fwd(x, torch.zeros(2, 5, 7), A, B, B)
    with pytest.raises(TypeError, match="delta"):
        ssm.ssm_scan_fwd(x, torch.zeros(2, 5, 8, dtype=bf), A, B, B)
    with pytest.raises(ValueError, match="B"):
        ssm.ssm_scan_fwd(x, x, A, torch.zeros(2, 5, 8), B)
    with pytest.raises(ValueError, match="last_state"):
        ssm.ssm_scan_fwd(x, x, A, B, B, last_state=torch.zeros(2, 8, 8))
    with pytest.raises(TypeError, match="D"):
        ssm.ssm_scan_fwd(x, x, A, B, B, D=torch.zeros(8, dtype=bf))
    with pytest.raises(ValueError, match="initial_state"):
        ssm.ssm_scan_fwd_from(x, x, A, B, B, initial_state=torch.zeros(2, 8))
    with pytest.raises(ValueError, match="dout"):
        ssm.ssm_scan_bwd(x, x, A, B, B, dout=torch.zeros(2, 4, 8))
    with pytest.raises(ValueError, match="B"):
        ssm.ssm_state_update(torch.zeros(2, 8, 16), x[:, 0], x[:, 0], A, torch.zeros(2, 8), torch.zeros(2, 16))
    with pytest.raises(ValueError, match="conv_state_in"):
        ssm.ssm_conv1d_fwd(x, torch.zeros(8, 4), conv_state_in=torch.zeros(2, 8, 3))
    with pytest.raises(TypeError, match="conv_state"):
        ssm.ssm_conv1d_update(torch.zeros(2, 8, 4, dtype=bf), x[:, 0], torch.zeros(8, 4))
    xs = torch.zeros(2, 5, 4, 64, dtype=bf)
    Bs = torch.zeros(2, 5, 2, 128, dtype=bf)
    with pytest.raises(ValueError, match="dt"):
        ssm.ssm_ssd_fwd(xs, torch.zeros(2, 5, 3, dtype=bf), torch.zeros(4), Bs, Bs)
    with pytest.raises(ValueError, match="D"):
        ssm.ssm_ssd_fwd(xs, torch.zeros(2, 5, 4, dtype=bf), torch.zeros(4), Bs, Bs, D=torch.zeros(4))
    with pytest.raises(ValueError, match="state"):
        ssm.ssm_ssd_state_update(torch.zeros(2, 4, 64, 64), xs[:, 0], torch.zeros(2, 4, dtype=bf), torch.zeros(4),
                                 Bs[:, 0], Bs[:, 0])
    with pytest.raises(ValueError, match="b"):
        ssm.ssm_affine_exclusive_scan(torch.zeros(5), torch.zeros(4))
    # consistent tensors pass the checks; these CPU tensors then fail the device check
    with pytest.raises(ValueError, match="GPU"):
        ssm.ssm_scan_fwd(x, x, A, B, B, D=torch.zeros(8, dtype=f32))
