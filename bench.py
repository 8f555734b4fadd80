"""Benchmark of libssmscan on one MI355X.

Default: the Mamba-2.8B-like layer scan (batch 8, d_inner 5120, d_state 16,
seqlen 2048; bf16 x/delta/z/B/C, fp32 state, softplus(delta + bias) fused,
D skip and SiLU(z) gate on, fp32 out).  One step = one ssm_scan_fwd call over
the whole batch with inputs resident in HBM.  Prints ONE JSON line:

  value       GB/s of algorithmic traffic (x, delta, z, B, C read once + out
              written once) over the K timed steps;
  roofline    the scan kernel against its binding ceiling, the VALU rate for
              its instruction mix (24 SIMD-cycles per wavefront of 64 state
              updates), with the plain fp32 FMA rate and the HBM fraction
              beside it;
  cpu_baseline the fp64 oracle on the host cores over the same workload;
  decode      512 consecutive ssm_state_update steps at batch 256, d_inner 8192:
              tokens/s (the second half of the metric).
  conv1d, backward, zoh, ssd
              the other operations on the layer's shape, each timed on its own
              (the backward and the Mamba-2 scan also on a long single-row
              sequence, in the planner's time chunks and in one chunk).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--out-dtype f32|bf16] [--no-cpu-baseline] [--no-decode]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, AMD spec
SIMDS, CLOCK_HZ = 256 * 4, 2.4e9  # 256 CUs x 4 SIMD16 at the 2.4 GHz peak engine clock
# fp32 FMA rate without packed-FP32 instructions (the build disables them):
# a wave64 VALU instruction occupies a SIMD16 for 4 cycles
FMA_PEAK_TFLOPS = SIMDS * 16 * 2 * CLOCK_HZ / 1e12
FLOPS_PER_STATE_UPDATE = 7       # mul (dt*A), exp, mul (dt*x*B), FMA (update, 2), FMA (readout, 2)
# The instruction-mix ceiling of one state update: four 4-cycle VALU
# instructions plus one v_exp_f32, which occupies the VALU for 8 cycles
# (measured: it does not overlap other VALU work), so 24 SIMD-cycles per
# wavefront of 64 updates.
CYCLES_PER_WAVE_UPDATE = 24
MIX_PEAK_TFLOPS = SIMDS * CLOCK_HZ * 64 / CYCLES_PER_WAVE_UPDATE * FLOPS_PER_STATE_UPDATE / 1e12


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(key):
    """HBM bytes per launch recorded from the FETCH_SIZE / WRITE_SIZE counters
    (scaled by a plain copy's reading) in profiles/*.md, or None when no record
    exists for `key` or the kernel source has changed since it was taken."""
    import glob
    from sequence_scan_amd import build as lib_build
    sha = lib_build.kernel_source_sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for row in f:
                if row.startswith("traffic-record: "):
                    rec = json.loads(row[len("traffic-record: "):])
                    if rec.get("kernel_source_sha256") == sha and key in rec:
                        return rec[key]["hbm_bytes"]
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="mamba2p8b",
                    choices=["mamba2p8b", "mamba130m", "long_dna", "tiny_fp32", "decode", "copy", "ssd"])
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-conv", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-ssd", action="store_true")
    ap.add_argument("--no-zoh", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=512)
    ap.add_argument("--plan", default=None, help="states_per_wave,chunk_len (tuning only)")
    return ap.parse_args()


def scan_case(name, out_dtype, plan_arg):
    import torch

    import sequence_scan_amd as ssm
    import workloads

    cfg = workloads.SCAN_CONFIGS[name]
    t0 = time.time()
    inp = workloads.scan_inputs(cfg, seed=0)
    log(f"generated {name} inputs in {time.time() - t0:.1f}s")
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dev = {}
    for k, v in inp.items():
        if k == "dtype":
            continue
        t = torch.from_numpy(v)
        if k in ("x", "delta", "z", "B", "C"):
            t = t.to(tdt)
        dev[k] = t.cuda()
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = torch.empty((cfg.batch, cfg.seqlen, cfg.d_inner), dtype=odt, device="cuda")
    last = torch.empty((cfg.batch, cfg.d_inner, cfg.d_state), dtype=torch.float32, device="cuda")
    plan = None
    if plan_arg:
        ns, cl = plan_arg.split(",")
        plan = {"states_per_wave": int(ns), "chunk_len": int(cl)}

    def run():
        ssm.ssm_scan_fwd(dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"],
                         dev["delta_bias"], softplus=True, out=out, last_state=last, plan=plan)

    nbytes = workloads.scan_algorithmic_bytes(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state, cfg.dtype, out_dtype)
    return cfg, inp, run, nbytes, plan


def capture_graph(fn):
    """fn's launches captured in a HIP graph (torch.cuda.CUDAGraph), after one
    warm-up call on a side stream."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def settle(run, seconds=0.05):
    """Run `run` back to back for about `seconds` (synchronising every ~2 ms of work)
    before a leg is timed.  The GPU raises its shader clock over the first tens of
    milliseconds of sustained load (on MI355X from about 2.1 to 2.4 GHz), so a leg
    timed right after an idle stretch would time the ramp instead of the sustained
    rate."""
    import torch
    torch.cuda.synchronize()
    t = time.perf_counter()
    run()
    torch.cuda.synchronize()
    batch = max(1, int(0.002 / max(time.perf_counter() - t, 1e-6)))
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            run()
        torch.cuda.synchronize()


def time_steps(run, steps, warmup):
    import torch
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return e0.elapsed_time(e1) / steps, wall


def per_launch_ms(run, reps, flush_bytes=0):
    """Average duration of one call, events around each call on the launch stream;
    with flush_bytes > 0 a buffer that size is overwritten before each call
    (outside the events) so the call starts with a cold last-level cache."""
    import torch
    buf = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda") if flush_bytes else None
    times = []
    for _ in range(reps):
        if buf is not None:
            buf.fill_(1.0)
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        run()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    times.sort()
    return sum(times) / len(times), times[len(times) // 2], times[0]


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo (None where it is not readable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, inp):
    import oracle
    nthreads = oracle.default_threads()
    t0 = time.perf_counter()
    oracle.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["delta_bias"],
                    softplus=True, nthreads=nthreads, return_state=False)
    return time.perf_counter() - t0, nthreads


def decode_case(steps):
    import torch

    import sequence_scan_amd as ssm
    import workloads

    cfg = workloads.DECODE_CONFIG
    t0 = time.time()
    inp = workloads.decode_inputs(cfg, seed=0, steps=steps)
    log(f"generated decode inputs ({steps} steps) in {time.time() - t0:.1f}s")
    dev = {}
    for k, v in inp.items():
        if k == "dtype":
            continue
        t = torch.from_numpy(v).cuda()
        if k in ("x", "delta", "z", "B", "C"):
            t = t.to(torch.bfloat16)  # exact: the values are bf16-representable
        dev[k] = t
    del inp
    state = torch.zeros((cfg.batch, cfg.d_inner, cfg.d_state), dtype=torch.float32, device="cuda")
    out = torch.empty((steps, cfg.batch, cfg.d_inner), dtype=torch.float32, device="cuda")

    def run_all():
        for s in range(steps):
            ssm.ssm_state_update(state, dev["x"][s], dev["delta"][s], dev["A"], dev["B"][s], dev["C"][s], dev["D"],
                                 dev["z"][s], dev["delta_bias"], softplus=True, out=out[s])

    run_all()  # warm-up pass (state then continues; the timing does not depend on values)
    torch.cuda.synchronize()
    state.zero_()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    run_all()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    per_step_bytes = workloads.decode_algorithmic_bytes(cfg.batch, cfg.d_inner, cfg.d_state, "bf16", "f32")
    step_ms = ms / steps
    return {
        "workload": f"decode batch {cfg.batch}, d_inner {cfg.d_inner}, d_state 16, {steps} steps, bf16 in, fp32 state/out",
        "tokens_per_s": cfg.batch * steps / (ms / 1e3),
        "us_per_step": step_ms * 1e3,
        "GBps_incl_state": per_step_bytes / (step_ms / 1e3) / 1e9,
        "hbm_frac_incl_state": per_step_bytes / (step_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
    }


def conv_case(batch, seqlen, d_inner, reps=20):
    """The conv1d front-end on a layer's shape: prefill (bf16 in, bf16 out, the
    scan's input) and one decode step at batch 256, d_inner 8192."""
    import torch

    import sequence_scan_amd as ssm
    import workloads

    inp = workloads.conv_inputs(batch, seqlen, d_inner, 4, "bf16", seed=0, with_state=True)
    x = torch.from_numpy(inp["x"]).to(torch.bfloat16).cuda()
    w = torch.from_numpy(inp["weight"]).cuda()
    b = torch.from_numpy(inp["bias"]).cuda()
    st = torch.from_numpy(inp["conv_state"]).to(torch.bfloat16).cuda()
    st_out = torch.empty_like(st)
    out = torch.empty_like(x)
    run = lambda: ssm.ssm_conv1d_fwd(x, w, b, conv_state_in=st, out=out, conv_state_out=st_out)
    settle(run)
    avg, _ = time_steps(run, reps, 3)  # back-to-back calls, events around the loop
    nbytes = workloads.conv_algorithmic_bytes(batch, seqlen, d_inner, 4, "bf16", "bf16")
    res = {"workload": f"conv1d prefill batch {batch}, seqlen {seqlen}, d_inner {d_inner}, d_conv 4, bf16 in/out, SiLU",
           "us_per_call": round(avg * 1e3, 2), "timing": "back-to-back calls (prefill kernel + cache kernel)",
           "bytes_per_call": nbytes,
           "GBps": round(nbytes / (avg / 1e3) / 1e9, 1), "hbm_frac": round(nbytes / (avg / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
    del x, out, inp
    dcfg = workloads.DECODE_CONFIG
    dinp = workloads.conv_inputs(dcfg.batch, 1, dcfg.d_inner, 4, "bf16", seed=1, with_state=True)
    xs = torch.from_numpy(dinp["x"][:, 0]).to(torch.bfloat16).cuda()
    ws = torch.from_numpy(dinp["weight"]).cuda()
    bs = torch.from_numpy(dinp["bias"]).cuda()
    cache = torch.from_numpy(dinp["conv_state"]).to(torch.bfloat16).cuda()
    dout = torch.empty_like(xs)
    step = lambda: ssm.ssm_conv1d_update(cache, xs, ws, bs, out=dout)
    settle(step)
    eager, _ = time_steps(step, 200, 10)  # 200 consecutive steps, events around the loop
    # The step's kernel takes a few microseconds, less than a Python call costs,
    # so the steps are also captured in a HIP graph and replayed: that time is
    # the GPU's.
    nsteps = 200
    g = capture_graph(lambda: [step() for _ in range(nsteps)])
    settle(g.replay)
    gms, _ = time_steps(g.replay, 3, 1)
    davg = gms / nsteps
    e = dcfg.batch * dcfg.d_inner
    dbytes = e * (2 * 4 * 2 + 2 + 2)  # cache read + written (4 bf16), x read, out written
    res["decode_step"] = {"workload": f"conv1d decode step batch {dcfg.batch}, d_inner {dcfg.d_inner}, bf16",
                          "us_per_step": round(davg * 1e3, 2), "timing": f"HIP graph of {nsteps} steps",
                          "us_per_step_eager": round(eager * 1e3, 2), "bytes_per_step": dbytes,
                          "GBps": round(dbytes / (davg / 1e3) / 1e9, 1)}
    return res


def backward_case(cfg, steps=5):
    """ssm_scan_bwd on the layer's shape (bf16 inputs and gradients, all optional
    inputs), timed as back-to-back calls."""
    import torch

    import sequence_scan_amd as ssm
    import workloads

    inp = workloads.scan_inputs(cfg, seed=0)
    t = {k: (torch.from_numpy(v).to(torch.bfloat16) if k in ("x", "delta", "z", "B", "C") else torch.from_numpy(v)).cuda()
         for k, v in inp.items() if k != "dtype"}
    del inp
    dout = torch.randn(t["x"].shape, device="cuda").to(torch.bfloat16)
    run = lambda: ssm.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                                   softplus=True, dout=dout)
    settle(run, 0.1)
    ms, _ = time_steps(run, steps, 2)
    # VALU cycles per wavefront state update: the checkpoint forward (3 VALU +
    # exp = 20), the tile's forward again with the readout (4 + exp = 24), the
    # reverse step (11 VALU + exp = 52) and the lane reductions of dB, dC (~12)
    cyc = 20 + 24 + 52 + 12
    updates = cfg.batch * cfg.seqlen * cfg.d_inner * cfg.d_state
    floor_us = updates / 64 * cyc / (SIMDS * CLOCK_HZ) * 1e6
    del t, dout
    return {"workload": f"ssm_scan_bwd {cfg.name}: batch {cfg.batch}, seqlen {cfg.seqlen}, d_inner {cfg.d_inner}, "
                        "bf16 inputs and gradients, softplus, D, z",
            "us_per_call": round(ms * 1e3, 1), "alu_floor_us": round(floor_us, 1),
            "alu_frac": round(floor_us / (ms * 1e3), 4), "long_sequence": backward_long_case()}


def backward_long_case():
    """ssm_scan_bwd on the long single-row workload (batch 1, 32 channel blocks): the
    planner's time chunks against one chunk.  Inputs are drawn on the GPU (seeded)."""
    import torch

    import sequence_scan_amd as ssm
    import workloads

    cfg = workloads.SCAN_CONFIGS["long_dna"]
    sh = (cfg.batch, cfg.seqlen, cfg.d_inner)
    gen = torch.Generator(device="cuda").manual_seed(7)

    def draw(shape, scale=1.0, shift=0.0, uniform=False):
        out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        flat = out.view(-1)
        for i in range(0, flat.numel(), 1 << 28):
            n = min(1 << 28, flat.numel() - i)
            r = torch.rand(n, generator=gen, device="cuda") if uniform else torch.randn(n, generator=gen, device="cuda")
            flat[i:i + n] = (r * scale + shift).to(torch.bfloat16)
        return out

    x, z, dout = draw(sh), draw(sh), draw(sh)
    dl = draw(sh, 4.605, -6.907, uniform=True)   # softplus^-1 of steps in [1e-3, 0.1]
    B, C = draw((cfg.batch, cfg.seqlen, cfg.d_state)), draw((cfg.batch, cfg.seqlen, cfg.d_state))
    A = (-torch.arange(1, cfg.d_state + 1, dtype=torch.float32, device="cuda")).repeat(cfg.d_inner, 1).contiguous()
    D = torch.ones(cfg.d_inner, device="cuda")
    bias = torch.zeros(cfg.d_inner, device="cuda")
    plan = ssm.ssm_scan_bwd_plan_query(*sh)
    res = {"workload": f"ssm_scan_bwd {cfg.name}: batch {cfg.batch}, seqlen {cfg.seqlen}, d_inner {cfg.d_inner}, "
                       "bf16 inputs and gradients, softplus, D, z", "plan": plan}
    for key, p in (("us_per_call", None), ("one_chunk_us_per_call",
                                           {"states_per_wave": 4, "chunk_len": cfg.seqlen})):
        run = lambda: ssm.ssm_scan_bwd(x, dl, A, B, C, D, z, bias, softplus=True, dout=dout, plan=p)
        settle(run, 0.1)
        ms, _ = time_steps(run, 3, 1)
        res[key] = round(ms * 1e3, 1)
    return res


def zoh_case(cfg, run_dt_ms, reps=20):
    """The scan with the exact zero-order-hold input coefficient (SSM_ZOH) on the
    layer's shape, timed as back-to-back calls, beside the dt coefficient's time."""
    import torch

    import sequence_scan_amd as ssm
    import workloads

    inp = workloads.scan_inputs(cfg, seed=0)
    t = {k: (torch.from_numpy(v).to(torch.bfloat16) if k in ("x", "delta", "z", "B", "C") else torch.from_numpy(v)).cuda()
         for k, v in inp.items() if k != "dtype"}
    del inp
    out = torch.empty(t["x"].shape, dtype=torch.float32, device="cuda")
    run = lambda: ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                                   out=out, zoh=True)
    settle(run)
    ms, _ = time_steps(run, reps, 3)
    return {"workload": f"{cfg.name} scan with SSM_ZOH (exact zero-order-hold input coefficient)",
            "us_per_call": round(ms * 1e3, 1), "dt_coefficient_us_per_call": round(run_dt_ms * 1e3, 1),
            "ratio": round(ms / run_dt_ms, 3)}


def ssd_case(reps=20, decode_steps=64):
    """The Mamba-2 (SSD) scan on its layer's shape (bf16 in, fp32 out, softplus,
    D, z), timed as back-to-back calls, against the HBM roofline (algorithmic
    bytes) with the matrix-core work beside it; and its decode step at batch 64."""
    import torch

    import sequence_scan_amd as ssm
    import workloads

    cfg = workloads.SSD_CONFIGS["mamba2_2p7b"]
    inp = workloads.ssd_inputs(cfg, seed=0)
    t = {k: (torch.from_numpy(v).to(torch.bfloat16) if k in ("x", "dt", "z", "B", "C") else torch.from_numpy(v)).cuda()
         for k, v in inp.items() if k != "dtype"}
    del inp
    out = torch.empty(t["x"].shape, dtype=torch.float32, device="cuda")
    run = lambda: ssm.ssm_ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["z"], t["dt_bias"], out=out)
    settle(run)
    ms, _ = time_steps(run, reps, 3)
    B_, L_, H_, P_, G_, N_ = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.d_state
    nbytes = workloads.ssd_algorithmic_bytes(B_, L_, H_, P_, G_, N_, "bf16", "f32")
    # algorithmic multiply-adds of the chunked form per (batch row, head, 64-step
    # chunk): C B^T (Q Q N), W X (Q Q P), C S^T (Q N P), the state update (Q P N)
    Q = 64
    macs = B_ * H_ * ((L_ + Q - 1) // Q) * (Q * Q * N_ + Q * Q * P_ + 2 * Q * N_ * P_)
    gbs = nbytes / (ms / 1e3) / 1e9
    tflops = 2 * macs / (ms / 1e3) / 1e12
    del t, out
    # decode step at batch 64
    dcfg = workloads.SsdConfig("mamba2_2p7b_decode", 64, decode_steps, H_, P_, G_, N_)
    dinp = workloads.ssd_inputs(dcfg, seed=1)
    dv = {k: (torch.from_numpy(v).to(torch.bfloat16) if k in ("x", "dt", "z", "B", "C") else torch.from_numpy(v)).cuda()
          for k, v in dinp.items() if k != "dtype"}
    del dinp
    steps = [{k: (v[:, s].contiguous() if k in ("x", "dt", "z", "B", "C") else v) for k, v in dv.items()}
             for s in range(decode_steps)]
    state = torch.zeros((64, H_, P_, N_), device="cuda")
    dout = torch.empty((64, H_, P_), dtype=torch.float32, device="cuda")

    def run_decode():
        for sv in steps:
            ssm.ssm_ssd_state_update(state, sv["x"], sv["dt"], sv["A"], sv["B"], sv["C"], sv["D"], sv["z"],
                                     sv["dt_bias"], out=dout)
    settle(run_decode)
    dms, _ = time_steps(run_decode, 2, 1)
    step_ms = dms / decode_steps
    step_bytes = 64 * H_ * P_ * (2 * 4 * N_ + 2 * 2 + 4) + 64 * (H_ * 2 + 2 * G_ * N_ * 2)
    return {"workload": f"ssm_ssd_fwd {cfg.name}: {cfg.description}; batch {B_}, seqlen {L_}, bf16 in, fp32 out, "
                        "softplus, D, z",
            "us_per_call": round(ms * 1e3, 1), "bytes_per_call": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("ssd_mamba2_2p7b")},
            "mfma": {"algorithmic_tflops": round(tflops, 1), "peak_bf16_tflops": 2500.0,
                     "frac": round(tflops / 2500.0, 4), "macs_per_call": macs},
            "decode_step": {"workload": f"ssm_ssd_state_update batch 64, {H_} heads x {P_}, d_state {N_}, bf16 in",
                            "us_per_step": round(step_ms * 1e3, 2), "bytes_per_step": step_bytes,
                            "GBps": round(step_bytes / (step_ms / 1e3) / 1e9, 1)},
            "long_sequence": ssd_long_case()}


def ssd_long_case():
    """ssm_ssd_fwd on one long row: the long workload's length and 2048 channels as 32
    Mamba-2 heads of 64 (d_state 128, one B/C group), in the planner's time chunks and
    in one chunk.  Inputs are drawn on the GPU (seeded)."""
    import torch

    import sequence_scan_amd as ssm
    import workloads

    L, H, P, N = workloads.SCAN_CONFIGS["long_dna"].seqlen, 32, 64, 128
    gen = torch.Generator(device="cuda").manual_seed(8)

    def draw(shape, scale=1.0, shift=0.0, uniform=False):
        out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        flat = out.view(-1)
        for i in range(0, flat.numel(), 1 << 28):
            n = min(1 << 28, flat.numel() - i)
            r = torch.rand(n, generator=gen, device="cuda") if uniform else torch.randn(n, generator=gen, device="cuda")
            flat[i:i + n] = (r * scale + shift).to(torch.bfloat16)
        return out

    x, z = draw((1, L, H, P)), draw((1, L, H, P))
    dt = draw((1, L, H), 4.605, -6.907, uniform=True)   # softplus^-1 of steps in [1e-3, 0.1]
    B, C = draw((1, L, 1, N)), draw((1, L, 1, N))
    A = -(torch.rand(H, generator=gen, device="cuda") * 2.0 + 0.5)
    D = torch.ones(H * P, device="cuda")
    bias = torch.zeros(H, device="cuda")
    out = torch.empty((1, L, H, P), device="cuda")
    plan = ssm.ssm_ssd_plan_query(1, L, H, P, 1, N)
    res = {"workload": f"ssm_ssd_fwd: batch 1, seqlen {L}, {H} heads x {P}, d_state {N}, one B/C group, bf16 in, "
                       "fp32 out, softplus, D, z", "plan": plan}
    for key, p in (("us_per_call", None), ("one_chunk_us_per_call", {"chunk_len": L})):
        run = lambda: ssm.ssm_ssd_fwd(x, dt, A, B, C, D, z, bias, out=out, plan=p)
        settle(run, 0.1)
        ms, _ = time_steps(run, 3, 1)
        res[key] = round(ms * 1e3, 1)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              "(rows shard over GPUs with no communication; run one process per GPU).", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    import sequence_scan_amd as ssm
    ssm.library()

    if args.workload == "copy":
        # a plain device-to-device copy of known size: the reference point for
        # the hardware byte counters and the achievable streaming bandwidth
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        ms, _ = time_steps(lambda: dst.copy_(src), args.steps, args.warmup)
        nbytes = 2 * n * 4
        print(json.dumps({"metric": "device copy bandwidth (read + write)", "value": round(nbytes / (ms / 1e3) / 1e9, 1),
                          "unit": "GB/s", "bytes_per_copy": nbytes, "ms_per_copy": round(ms, 4), "n_gpus": 1}), flush=True)
        return

    if args.workload == "ssd":
        d = ssd_case(args.steps)
        print(json.dumps({"metric": "Mamba-2 SSD scan GB/s", "value": d["roofline"]["achieved"], "unit": "GB/s",
                          "n_gpus": 1, "higher_is_better": True, "ssd": d}), flush=True)
        return

    if args.workload == "decode":
        d = decode_case(args.decode_steps)
        print(json.dumps({"metric": "decode tokens/sec at batch 256", "value": round(d["tokens_per_s"], 1),
                          "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True, "decode": d}), flush=True)
        return

    cfg, inp, run, nbytes, plan = scan_case(args.workload, args.out_dtype, args.plan)
    plan_used = plan or ssm.ssm_scan_plan(cfg.batch, cfg.seqlen, cfg.d_inner)
    log(f"plan {plan_used}; algorithmic bytes {nbytes}")
    # The shader clock needs tens of milliseconds of sustained load to reach its
    # steady rate: run the step back to back for 50 ms first (untimed), so that
    # the result does not depend on how few warm-up steps a caller asks for.
    settle(run)
    ms, wall = time_steps(run, args.steps, args.warmup)
    gbs = nbytes / (ms / 1e3) / 1e9
    log(f"{args.steps} steps: {ms * 1e3:.1f} us/step (events), wall {wall * 1e3:.1f} ms, {gbs:.1f} GB/s")

    # dominant kernel: with one time chunk the whole step is one launch of the scan
    # kernel, and back-to-back launches on the stream abut, so its average launch
    # duration is the timed region's time per step (events on the launch stream);
    # chunked plans launch three kernels per step and report the whole call
    single_launch = plan_used.get("n_chunks", 1) in (1, None)
    i_avg, i_med, i_min = per_launch_ms(run, max(10, args.steps))
    k_avg = ms if single_launch else i_avg
    c_avg, c_med, c_min = per_launch_ms(run, 10, flush_bytes=1 << 30)
    states = cfg.batch * cfg.seqlen * cfg.d_inner * cfg.d_state
    tflops = states * FLOPS_PER_STATE_UPDATE / (k_avg / 1e3) / 1e12
    k_gbs = nbytes / (k_avg / 1e3) / 1e9
    traffic = None
    if single_launch and args.out_dtype == "f32" and not args.plan:
        traffic = measured_traffic(f"scan_{cfg.name}")
    roofline = {
        "bound": "alu",
        "achieved": round(tflops, 2),
        "peak": round(MIX_PEAK_TFLOPS, 2),
        "unit": "TFLOP/s",
        "frac": round(tflops / MIX_PEAK_TFLOPS, 4),
        "traffic": traffic,
        "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, each scaled by a plain copy's reading)",
        "kernel": "scan_chunk_kernel (pass B)" if single_launch else "ssm_scan_fwd (all passes)",
        "flops_per_state_update": FLOPS_PER_STATE_UPDATE,
        "peak_basis": "1024 SIMDs x 2.4 GHz x 64 lanes / 24 cycles per wavefront state update x 7 flops",
        "fp32_fma_peak": round(FMA_PEAK_TFLOPS, 2),
        "fp32_fma_frac": round(tflops / FMA_PEAK_TFLOPS, 4),
        "state_updates_per_launch": states,
        "avg_launch_us": round(k_avg * 1e3, 2),
        "launch_timing": "timed region (back-to-back launches)" if single_launch else "single calls",
        "isolated_call_us": round(i_avg * 1e3, 2),
        "hbm": {"achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(k_gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": nbytes},
        "cold_llc_us": {"avg": round(c_avg * 1e3, 2), "median": round(c_med * 1e3, 2), "min": round(c_min * 1e3, 2)},
    }
    line = {
        "metric": "selective-scan GB/s and % HBM peak (prefill); decode tokens/sec at batch 256",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle_s": 0.05,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; shapes and distributions of the workload table)",
        "config": {"workload": f"{cfg.name}: {cfg.description}", "batch": cfg.batch, "seqlen": cfg.seqlen,
                   "d_inner": cfg.d_inner, "d_state": cfg.d_state, "in_dtype": cfg.dtype,
                   "out_dtype": args.out_dtype, "plan": plan_used},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host cores")
        secs, cores = cpu_baseline(cfg, inp)
        line["cpu_baseline"] = {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": cores,
                                "kind": "oracle", "seconds": round(secs, 2), "cpu": cpu_model(),
                                "sample": f"the full {cfg.name} workload (every row and step), fp64"}
    del inp
    if not args.no_decode and args.workload == "mamba2p8b":
        line["decode"] = decode_case(args.decode_steps)
    if not args.no_conv and args.workload == "mamba2p8b":
        line["conv1d"] = conv_case(cfg.batch, cfg.seqlen, cfg.d_inner)
    if not args.no_backward and args.workload == "mamba2p8b":
        line["backward"] = backward_case(cfg)
    if not args.no_zoh and args.workload == "mamba2p8b":
        line["zoh"] = zoh_case(cfg, ms)
    if not args.no_ssd and args.workload == "mamba2p8b":
        line["ssd"] = ssd_case()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
