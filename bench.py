"""Benchmark of libssmscan on one MI355X.

Default: the Mamba-2.8B-like layer scan (batch 8, d_inner 5120, d_state 16,
seqlen 2048; bf16 x/delta/z/B/C, fp32 state, softplus(delta + bias) fused,
D skip and SiLU(z) gate on, fp32 out).  One step = one ssm_scan_fwd call over
the whole batch with inputs resident in HBM.  Prints ONE JSON line:

  value       GB/s of algorithmic traffic (x, delta, z, B, C read once + out
              written once) over the K timed steps;
  roofline    the scan kernel against the HBM roofline (8 TB/s), with the
              ceiling that binds it beside it: the VALU issue rate of its
              instruction mix (SIMD-cycles per wavefront state update, read
              from the VALU probe's record in profiles/);
  cpu_baseline the fp64 oracle on the host cores over the same workload, and
              on one thread over the tiny and Mamba-130M-like workloads;
  legs        the other scan workloads (tiny, Mamba-130M-like, long DNA-like)
              and the layer with bf16 out, each against both ceilings;
  valu_probe  the issue-rate probe, run live (cycles per instruction);
  decode      512 consecutive ssm_state_update steps at batch 256, d_inner 8192:
              tokens/s (the second half of the metric).
  conv1d, backward, zoh, ssd
              the other operations on the layer's shape, each timed on its own
              (the backward and the Mamba-2 scan also on a long single-row
              sequence, in the planner's time chunks and in one chunk).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--out-dtype f32|bf16] [--no-cpu-baseline] [--no-decode] [--no-legs]
  --workload valu   only the VALU issue-rate probe
  --workload copy   only the 1 GiB streaming legs: torch's copy (the byte counters'
                    reference) and the streaming probe's copy and read
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
FP32_PEAK_TFLOPS = 157.3         # MI355X published fp32 vector peak (packed-fp32 instructions)
# fp32 FMA rate without packed-FP32 instructions (the build disables them):
# a wave64 VALU instruction occupies a SIMD16 for 4 cycles
FMA_PEAK_TFLOPS = SIMDS * 16 * 2 * CLOCK_HZ / 1e12
FLOPS_PER_STATE_UPDATE = 7       # mul (dt*A), exp, mul (dt*x*B), FMA (update, 2), FMA (readout, 2)
# The instruction-mix ceiling of one state update (four VALU instructions and
# one v_exp_f32) is measured by the VALU probe leg (--workload valu) and read
# from its record in profiles/; MODEL_CYCLES_PER_WAVE_UPDATE (4 x 4 + 8, the
# per-instruction costs of the ISA's issue model) is used only when no record
# exists.
MODEL_CYCLES_PER_WAVE_UPDATE = 24.0
# transitions as powers of one exponential: 21 VALU instructions per 4 updates
# at ~2.2 cycles each, no transcendental
MODEL_POWERS_CYCLES_PER_WAVE_UPDATE = 21 / 4 * 2.2


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def read_record(tag, key=None):
    """The newest record line `<tag>: {json}` in profiles/*.md (for a traffic record,
    the one taken with the current kernel sources, by key), or None."""
    import glob
    sha = None
    if tag == "traffic-record":
        from sequence_scan_amd import build as lib_build
        sha = lib_build.kernel_source_sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for row in f:
                if row.startswith(tag + ": "):
                    rec = json.loads(row[len(tag) + 2:])
                    if sha is not None and rec.get("kernel_source_sha256") != sha:
                        continue
                    if key is None:
                        return rec
                    if key in rec:
                        return rec[key]
    return None


def measured_traffic(key):
    """HBM bytes per launch recorded from the FETCH_SIZE / WRITE_SIZE counters
    (scaled by a plain copy's reading) in profiles/*.md, or None when no record
    exists for `key` or the kernel source has changed since it was taken."""
    rec = read_record("traffic-record", key)
    return None if rec is None else rec["hbm_bytes"]


def mix_ceiling(powers=False):
    """(cycles per wavefront state update, where it comes from) for the scan's
    instruction mix: the VALU probe's record in profiles/, else the issue model.
    `powers`: the mix of the transitions formed as powers of one exponential,
    which the kernel runs where A[d, n] = (n + 1) A[d, 0] (every stated workload)."""
    rec = read_record("valu-record")
    key = "scan_powers_cycles_per_wave_update" if powers else "scan_mix_cycles_per_wave_update"
    if rec is not None and key in rec:
        return float(rec[key]), f"measured (profiles/ valu-record, {key})"
    return (MODEL_POWERS_CYCLES_PER_WAVE_UPDATE if powers else MODEL_CYCLES_PER_WAVE_UPDATE,
            "issue model (no valu-record in profiles/)")


def backward_cycles():
    """SIMD-cycles per wavefront state update of the backward on the workload's A,
    from the VALU probe's issue rates: the forward kernel's checkpoint pass (the
    powers update without its readout FMA: 17 of the 21 instructions per 4 updates),
    the tile's recompute with readout (one exponential per update: the probe's
    exponential mix), the reverse step (9 VALU per update) and the dB/dC lane sums
    (18 VALU per step for 4 updates), the last two at the VALU rate of a stream that
    carries exponentials (the exponential mix less its v_exp_f32, over its 4 VALU)."""
    powers, src = mix_ceiling(True)
    mix, _ = mix_ceiling(False)
    rec = read_record("valu-record")
    try:
        exp_c = float(rec["cycles"]["v_exp_f32"]["8"])
    except (TypeError, KeyError, ValueError):
        exp_c = 8.3
    valu_in_exp_stream = (mix - exp_c) / 4
    parts = {"checkpoint_pass": powers * 17 / 21, "recompute": mix, "reverse": 9 * valu_in_exp_stream,
             "lane_sums": 18 / 4 * valu_in_exp_stream}
    return sum(parts.values()), {k: round(v, 2) for k, v in parts.items()}, src


def alu_floor_us(updates, cycles):
    """Time of `updates` state updates at `cycles` SIMD-cycles per wavefront of 64,
    on every SIMD at the 2.4 GHz peak clock."""
    return updates / 64 * cycles / (SIMDS * CLOCK_HZ) * 1e6


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="mamba2p8b",
                    choices=["mamba2p8b", "mamba130m", "long_dna", "tiny_fp32", "decode", "copy", "ssd", "valu"])
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-conv", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-ssd", action="store_true")
    ap.add_argument("--no-zoh", action="store_true")
    ap.add_argument("--no-legs", action="store_true", help="skip the other scan workloads and the VALU probe")
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


def per_launch_ms(run, reps):
    """Average, median and minimum duration of one call, with events around each call
    on the launch stream and a synchronisation after it."""
    import torch
    times = []
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        run()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    times.sort()
    return sum(times) / len(times), times[len(times) // 2], times[0]


def cold_warm_ms(run, reps=20, flush_bytes=1 << 30):
    """Single calls with and without a cold cache, interleaved so both see the same
    clock history: before each cold call a 1 GiB buffer is read (summed) and the
    device synchronised, so the call starts with caches holding none of its data;
    each warm call follows the previous call directly.  Returns the medians and
    minima (ms).  The flush reads rather than writes, so no dirty lines are left to
    be written back during the timed call."""
    import torch
    buf = torch.ones(flush_bytes // 4, dtype=torch.float32, device="cuda")
    cold, warm = [], []
    for i in range(2 * reps):
        if i % 2 == 0:
            buf.sum()
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        run()
        e.record()
        torch.cuda.synchronize()
        (cold if i % 2 == 0 else warm).append(s.elapsed_time(e))
    del buf
    cold.sort()
    warm.sort()
    return {"cold_median": cold[reps // 2], "cold_min": cold[0], "warm_median": warm[reps // 2], "warm_min": warm[0]}


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
    copy_rec = read_record("copy-record")
    return {
        "workload": f"decode batch {cfg.batch}, d_inner {cfg.d_inner}, d_state 16, {steps} steps, bf16 in, fp32 state/out",
        "tokens_per_s": cfg.batch * steps / (ms / 1e3),
        "us_per_step": step_ms * 1e3,
        "GBps_incl_state": per_step_bytes / (step_ms / 1e3) / 1e9,
        "hbm_frac_incl_state": per_step_bytes / (step_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "frac_of_measured_copy": (round(per_step_bytes / (step_ms / 1e3) / 1e9 / copy_rec["GBps"], 4)
                                  if copy_rec else None),
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
    # single calls with a synchronisation after each: the workspace (about 840 MB)
    # is reused from the library's pool instead of being mapped again per call
    iso_avg, iso_med, _ = per_launch_ms(run, 5)
    cyc, parts, src = backward_cycles()
    updates = cfg.batch * cfg.seqlen * cfg.d_inner * cfg.d_state
    floor_us = alu_floor_us(updates, cyc)
    # a training step's scan: forward then backward, with the backward computing its
    # checkpoints again, against the forward keeping them (ssm_scan_fwd_ckpt) and the
    # backward reading them (ssm_scan_bwd_ckpt)
    args = (t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"])
    out = torch.empty(t["x"].shape, device="cuda")
    ck = torch.empty((ssm.ssm_scan_ckpt_bytes(cfg.batch, cfg.seqlen, cfg.d_inner),), dtype=torch.uint8, device="cuda")
    step = lambda: (ssm.ssm_scan_fwd_from(*args, out=out), ssm.ssm_scan_bwd(*args, softplus=True, dout=dout))
    step_ck = lambda: (ssm.ssm_scan_fwd_ckpt(*args, out=out, ckpt=ck),
                       ssm.ssm_scan_bwd(*args, softplus=True, dout=dout, ckpt=ck))
    fwd_ck = lambda: ssm.ssm_scan_fwd_ckpt(*args, out=out, ckpt=ck)
    bwd_ck = lambda: ssm.ssm_scan_bwd(*args, softplus=True, dout=dout, ckpt=ck)
    tr = {}
    for name, fn in (("forward_then_backward", step), ("forward_with_checkpoints_then_backward", step_ck),
                     ("forward_with_checkpoints", fwd_ck), ("backward_from_checkpoints", bwd_ck)):
        settle(fn, 0.05)
        tr[name + "_us"] = round(time_steps(fn, steps, 1)[0] * 1e3, 1)
    del t, dout, out, ck
    return {"workload": f"ssm_scan_bwd {cfg.name}: batch {cfg.batch}, seqlen {cfg.seqlen}, d_inner {cfg.d_inner}, "
                        "bf16 inputs and gradients, softplus, D, z",
            "us_per_call": round(ms * 1e3, 1), "isolated_call_us": {"avg": round(iso_avg * 1e3, 1),
                                                                    "median": round(iso_med * 1e3, 1)},
            "alu_floor_us": round(floor_us, 1), "alu_cycles_per_wave_update": round(cyc, 2),
            "alu_cycles_parts": parts, "alu_cycles_source": src,
            "alu_frac": round(floor_us / (ms * 1e3), 4),
            "training_step": dict(tr, checkpoint_bytes=ssm.ssm_scan_ckpt_bytes(cfg.batch, cfg.seqlen, cfg.d_inner)),
            "long_sequence": backward_long_case()}


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


def stream_case(steps, warmup):
    """1 GiB of fp32 copied by torch (the byte counters' reference), and copied and
    read by the streaming probe (csrc/stream_probe.hip): the achievable HBM rates
    for a read + write stream and a read-only stream."""
    import ctypes

    import torch

    from sequence_scan_amd import build as lib_build
    lib = ctypes.CDLL(lib_build.PROBE_LIB)
    lib.ssm_stream_probe_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_void_p]
    lib.ssm_stream_probe_launch.restype = ctypes.c_int
    n = 1 << 28
    nbytes = n * 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def probe(kind, out):
        rc = lib.ssm_stream_probe_launch(kind, src.data_ptr(), out.data_ptr(), n // 4, stream)
        if rc != 0:
            raise RuntimeError(f"stream probe launch failed: hip error {rc}")

    res = {"metric": "device streaming bandwidth", "unit": "GB/s", "buffer_bytes": nbytes, "n_gpus": 1,
           "steps": steps, "warmup": warmup}
    for name, fn, traffic in (("torch_copy", lambda: dst.copy_(src), 2 * nbytes),
                              ("probe_copy", lambda: probe(0, dst), 2 * nbytes),
                              ("probe_read", lambda: probe(1, sink), nbytes)):
        settle(fn)
        ms, _ = time_steps(fn, steps, warmup)
        res[name] = {"GBps": round(traffic / (ms / 1e3) / 1e9, 1), "ms": round(ms, 4), "bytes": traffic}
    res["value"] = res["probe_copy"]["GBps"]
    return res


def valu_probe_case(total_iters=16384):
    """SIMD-cycles per wave64 instruction of v_mul_f32, v_fma_f32, v_exp_f32, v_log_f32
    and v_rcp_f32, and per state update of the scan's instruction mix (two v_mul, two
    v_fma, one v_exp: kind 3 of csrc/valu_probe.hip), at 1 to 8 wavefronts per SIMD;
    also the update without its exponential, a v_mul with an SGPR operand, and
    exponential-only wavefronts beside FMA-only ones (kinds 6-8).
    cycles = launch duration x measured shader clock / instructions issued per SIMD;
    the clock is the median over wavefronts of d(s_memtime) / d(s_memrealtime) x 100 MHz."""
    import ctypes

    import numpy as np
    import torch

    from sequence_scan_amd import build as lib_build
    lib = ctypes.CDLL(lib_build.PROBE_LIB)
    lib.ssm_probe_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]
    lib.ssm_probe_launch.restype = ctypes.c_int
    lib.ssm_probe_ops_per_iter.argtypes = [ctypes.c_int]
    lib.ssm_probe_ops_per_iter.restype = ctypes.c_int
    names = {0: "v_mul_f32", 1: "v_fma_f32", 2: "v_exp_f32", 4: "v_log_f32", 5: "v_rcp_f32", 3: "scan_update",
             6: "scan_update_without_exp", 7: "v_mul_f32_sgpr_operand", 8: "exp_waves_beside_fma_waves",
             9: "scan_update_powers"}
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for kind in (0, 1, 2, 4, 5, 3, 6, 7, 8, 9):
        per = {}
        for wps in (1, 2, 3, 4, 8):
            blocks = 256 * wps            # workgroups of 4 wavefronts (one per SIMD)
            iters = max(1, total_iters // wps)
            sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
            stamps = torch.zeros(blocks * 16, dtype=torch.int64, device="cuda")

            def run():
                rc = lib.ssm_probe_launch(kind, blocks, iters, 0.37, sink.data_ptr(), stamps.data_ptr(), stream)
                if rc != 0:
                    raise RuntimeError(f"probe launch failed: hip error {rc}")
            settle(run, 0.05)
            ms, _ = time_steps(run, 5, 1)
            st = stamps.view(-1, 4).cpu().numpy().astype(np.float64)
            clk = float(np.median((st[:, 1] - st[:, 0]) / np.maximum(st[:, 3] - st[:, 2], 1.0))) * 100e6
            ops = wps * iters * lib.ssm_probe_ops_per_iter(kind)    # per SIMD
            per[str(wps)] = {"cycles": round(ms / 1e3 * clk / ops, 3), "clock_ghz": round(clk / 1e9, 3),
                             "ms": round(ms, 4)}
        res[names[kind]] = per
    best = min(v["cycles"] for k, v in res["scan_update"].items() if int(k) >= 2)
    best_pow = min(v["cycles"] for k, v in res["scan_update_powers"].items() if int(k) >= 2)
    return {"unit": "SIMD-cycles per wave64 instruction (scan_update*: per state update)",
            "method": "launch duration x measured shader clock / instructions issued per SIMD",
            "rates": res, "scan_mix_cycles_per_wave_update": best,
            "scan_powers_cycles_per_wave_update": best_pow}


def a_is_powers(A) -> bool:
    """Whether every row of A is (n + 1) * A[d, 0] exactly: the kernel then forms the
    transitions as powers of one exponential (the same check it makes per block)."""
    import numpy as np
    A = np.asarray(A, dtype=np.float32)
    return bool(np.all(A == np.arange(1, A.shape[1] + 1, dtype=np.float32)[None, :] * A[:, :1]))


def gpu_scan_inputs(cfg, seed=7, general_a=False):
    """Inputs of the same shape and distributions as workloads.scan_inputs, drawn on
    the GPU with torch's seeded generator (for timing only; parity tests use the
    workloads generator).  Step sizes: Delta* log-uniform in [dmin, dmax] per element
    and beta per channel, bias = log(expm1(beta)), delta = log(expm1(Delta*)) - bias."""
    import math

    import torch
    gen = torch.Generator(device="cuda").manual_seed(seed)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    shape = (cfg.batch, cfg.seqlen, cfg.d_inner)
    lo, hi = math.log(cfg.dmin), math.log(cfg.dmax)

    def normal(shp):
        out = torch.empty(shp, dtype=tdt, device="cuda")
        flat = out.view(-1)
        for i in range(0, flat.numel(), 1 << 28):
            n = min(1 << 28, flat.numel() - i)
            flat[i:i + n] = torch.randn(n, generator=gen, device="cuda").to(tdt)
        return out

    beta = torch.exp(lo + (hi - lo) * torch.rand(cfg.d_inner, generator=gen, device="cuda", dtype=torch.float64))
    bias = torch.log(torch.expm1(beta)).float()
    delta = torch.empty(shape, dtype=tdt, device="cuda")
    dflat = delta.view(-1, cfg.d_inner)
    rows = max(1, (1 << 28) // cfg.d_inner)
    for r in range(0, dflat.shape[0], rows):
        n = min(rows, dflat.shape[0] - r)
        tgt = torch.exp(lo + (hi - lo) * torch.rand((n, cfg.d_inner), generator=gen, device="cuda"))
        dflat[r:r + n] = (torch.log(torch.expm1(tgt)) - bias).to(tdt)
    if cfg.x_kind == "dna":
        W = torch.randn((4, cfg.d_inner), generator=gen, device="cuda")
        x = torch.empty(shape, dtype=tdt, device="cuda")
        xflat = x.view(-1, cfg.d_inner)
        for r in range(0, xflat.shape[0], rows):
            n = min(rows, xflat.shape[0] - r)
            tok = torch.randint(0, 4, (n,), generator=gen, device="cuda")
            xflat[r:r + n] = (W[tok] + 0.1 * torch.randn((n, cfg.d_inner), generator=gen, device="cuda")).to(tdt)
    else:
        x = normal(shape)
    if general_a:   # a general A < 0 per (channel, state), as a trained layer holds
        A = -torch.exp(torch.rand((cfg.d_inner, cfg.d_state), generator=gen, device="cuda") * 4.0 - 1.0)
    else:
        A = (-torch.arange(1, cfg.d_state + 1, dtype=torch.float32, device="cuda")).repeat(cfg.d_inner, 1).contiguous()
    return {"x": x, "delta": delta, "z": normal(shape), "B": normal((cfg.batch, cfg.seqlen, cfg.d_state)),
            "C": normal((cfg.batch, cfg.seqlen, cfg.d_state)), "A": A,
            "D": torch.ones(cfg.d_inner, device="cuda"), "delta_bias": bias}


def scan_leg(name, out_dtype, reps=20, gpu_inputs=False, general_a=False):
    """ssm_scan_fwd on workload `name` (default plan; softplus, D and z on), timed as
    back-to-back calls at the sustained clock, against the HBM roofline and the
    instruction-mix ceiling of the path the kernel takes.  `general_a` replaces the
    workload's A = -(n + 1) by a general A (the exponential path).  The tiny workload
    is launch-bound: its calls are also captured in a HIP graph and replayed, which
    gives the GPU's own time per call."""
    import torch

    import sequence_scan_amd as ssm
    import workloads
    cfg = workloads.SCAN_CONFIGS[name]
    if gpu_inputs or general_a:
        dev = gpu_scan_inputs(cfg, general_a=general_a)
    else:
        inp = workloads.scan_inputs(cfg, seed=0)
        tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        dev = {k: (torch.from_numpy(v).to(tdt) if k in ("x", "delta", "z", "B", "C") else torch.from_numpy(v)).cuda()
               for k, v in inp.items() if k != "dtype"}
        del inp
    powers = a_is_powers(dev["A"].cpu().numpy())
    cyc, cyc_src = mix_ceiling(powers)
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = torch.empty((cfg.batch, cfg.seqlen, cfg.d_inner), dtype=odt, device="cuda")
    last = torch.empty((cfg.batch, cfg.d_inner, cfg.d_state), dtype=torch.float32, device="cuda")
    run = lambda: ssm.ssm_scan_fwd(dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"],
                                   dev["delta_bias"], softplus=True, out=out, last_state=last)
    settle(run, 0.1)
    ms, _ = time_steps(run, reps, 3)
    nbytes = workloads.scan_algorithmic_bytes(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state, cfg.dtype, out_dtype)
    updates = cfg.batch * cfg.seqlen * cfg.d_inner * cfg.d_state
    res = {"workload": f"{name}: {cfg.description}; batch {cfg.batch}, seqlen {cfg.seqlen}, d_inner {cfg.d_inner}, "
                       f"{cfg.dtype} in, {out_dtype} out, softplus, D, z" + (", general A" if general_a else ""),
           "inputs": ("drawn on the GPU (same distributions" + (", A = -exp(U(-1, 3)) per (d, n))" if general_a
                                                                 else ")")) if (gpu_inputs or general_a)
                     else "workloads generator, seed 0",
           "transitions": "powers of one exponential" if powers else "one exponential per state",
           "alu_cycles_per_wave_update": cyc, "alu_cycles_source": cyc_src,
           "plan": ssm.ssm_scan_plan(cfg.batch, cfg.seqlen, cfg.d_inner), "bytes_per_call": nbytes}
    if name == "tiny_fp32":
        eager = ms
        n = 100
        g = capture_graph(lambda: [run() for _ in range(n)])
        settle(g.replay, 0.05)
        gms, _ = time_steps(g.replay, 5, 1)
        ms = gms / n
        res.update({"us_per_call_eager": round(eager * 1e3, 2), "timing": f"HIP graph of {n} calls, replayed"})
    else:
        res["timing"] = f"{reps} back-to-back calls"
    floor = alu_floor_us(updates, cyc)
    gbs = nbytes / (ms / 1e3) / 1e9
    res.update({"us_per_call": round(ms * 1e3, 2), "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                "alu_floor_us": round(floor, 2), "alu_frac": round(floor / (ms * 1e3), 4)})
    del dev, out, last
    return res


def cpu_single_thread():
    """The oracle on one host thread over the tiny and the Mamba-130M-like workloads."""
    import oracle
    import workloads
    res = {}
    for name in ("tiny_fp32", "mamba130m"):
        cfg = workloads.SCAN_CONFIGS[name]
        inp = workloads.scan_inputs(cfg, seed=0)
        t0 = time.perf_counter()
        oracle.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["delta_bias"],
                        softplus=True, nthreads=1, return_state=False)
        secs = time.perf_counter() - t0
        nbytes = workloads.scan_algorithmic_bytes(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state, cfg.dtype, "f32")
        res[name] = {"seconds": round(secs, 4), "GBps": round(nbytes / secs / 1e9, 5), "cores": 1}
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
        # a plain device-to-device copy of known size (torch's copy kernel): the
        # reference point for the hardware byte counters; beside it the streaming
        # probe's copy and read of the same buffer, the achievable HBM rates
        print(json.dumps(stream_case(args.steps, args.warmup)), flush=True)
        return

    if args.workload == "valu":
        d = valu_probe_case()
        print(json.dumps({"metric": "VALU issue rates (SIMD-cycles per wave64 instruction)",
                          "value": d["scan_mix_cycles_per_wave_update"], "unit": "cycles per wavefront state update",
                          "n_gpus": 1, "higher_is_better": False, "valu": d}), flush=True)
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
    powers = a_is_powers(inp["A"])
    cyc, cyc_src = mix_ceiling(powers)
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
    cw = cold_warm_ms(run)
    states = cfg.batch * cfg.seqlen * cfg.d_inner * cfg.d_state
    tflops = states * FLOPS_PER_STATE_UPDATE / (k_avg / 1e3) / 1e12
    k_gbs = nbytes / (k_avg / 1e3) / 1e9
    traffic = None
    if single_launch and args.out_dtype == "f32" and not args.plan:
        traffic = measured_traffic(f"scan_{cfg.name}")
    floor_us = alu_floor_us(states, cyc)
    copy_rec = read_record("copy-record")
    mix_peak = SIMDS * CLOCK_HZ * 64 / cyc * FLOPS_PER_STATE_UPDATE / 1e12
    roofline = {
        "bound": "hbm",
        "achieved": round(k_gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(k_gbs / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, each scaled by a plain copy's reading)",
        "kernel": "scan_chunk_kernel (pass B)" if single_launch else "ssm_scan_fwd (all passes)",
        "bytes_per_launch": nbytes,
        "avg_launch_us": round(k_avg * 1e3, 2),
        "launch_timing": "timed region (back-to-back launches)" if single_launch else "single calls",
        "isolated_call_us": round(i_avg * 1e3, 2),
        "frac_of_measured_copy": (round(k_gbs / copy_rec["GBps"], 4) if copy_rec else None),
        "measured_copy_GBps": copy_rec["GBps"] if copy_rec else None,
        "cold_cache_us": {k: round(v * 1e3, 2) for k, v in cw.items()},
        "cold_cache_timing": "single synchronised calls, cold (after a 1 GiB read) and warm interleaved",
        # The ceiling beside HBM is the VALU issue rate of the state update's
        # instruction mix: with the workload's A = -(n + 1) the kernel forms the
        # transitions as powers of one exponential (21 VALU instructions per 4
        # updates), with a general A one v_exp_f32 and four VALU per update.  The
        # kernel's traffic is ~1.02x the algorithmic bytes.
        "alu": {
            "transitions": "powers of one exponential" if powers else "one exponential per state",
            "cycles_per_wave_update": cyc,
            "cycles_source": cyc_src,
            "floor_us": round(floor_us, 2),
            "frac": round(floor_us / (k_avg * 1e3), 4),
            "achieved_tflops": round(tflops, 2),
            "mix_peak_tflops": round(mix_peak, 2),
            "flops_per_state_update": FLOPS_PER_STATE_UPDATE,
            "peak_basis": f"1024 SIMDs x 2.4 GHz x 64 lanes / {cyc} cycles per wavefront state update",
            "cycles_per_wave_update_with_exponentials": mix_ceiling(False)[0],
            "fp32_peak_tflops": FP32_PEAK_TFLOPS,
            "fp32_peak_frac": round(tflops / FP32_PEAK_TFLOPS, 4),
            "fp32_unpacked_fma_peak_tflops": round(FMA_PEAK_TFLOPS, 2),
            "state_updates_per_launch": states,
        },
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
        if args.workload == "mamba2p8b":
            log("timing the fp64 oracle on one host thread (tiny, Mamba-130M-like)")
            line["cpu_baseline"]["single_thread"] = cpu_single_thread()
    del inp
    full = args.workload == "mamba2p8b"
    if full and not args.no_legs:
        log("legs: the other scan workloads, VALU probe")
        line["legs"] = {
            "mamba2p8b_bf16_out": scan_leg("mamba2p8b", "bf16"),
            "mamba2p8b_general_A": scan_leg("mamba2p8b", "f32", general_a=True),
            "mamba130m": scan_leg("mamba130m", "f32"),
            "tiny_fp32": scan_leg("tiny_fp32", "f32"),
            "long_dna": scan_leg("long_dna", "f32", reps=5, gpu_inputs=True),
        }
        line["valu_probe"] = valu_probe_case()
    if not args.no_decode and full:
        line["decode"] = decode_case(args.decode_steps)
    if not args.no_conv and full:
        line["conv1d"] = conv_case(cfg.batch, cfg.seqlen, cfg.d_inner)
    if not args.no_backward and full:
        line["backward"] = backward_case(cfg)
    if not args.no_zoh and full:
        line["zoh"] = zoh_case(cfg, ms)
    if not args.no_ssd and full:
        line["ssd"] = ssd_case()
    print(json.dumps(line), flush=True)

if __name__ == "__main__":
    main()
