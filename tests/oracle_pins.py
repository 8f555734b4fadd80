"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``pin_*`` function takes a bound oracle (``oracle.OracleLib``) and raises
AssertionError when the oracle disagrees with an independent statement of the
result: a brute-force formula computed here with numpy (never the oracle's
recurrence), a closed form, a special case, an invariant, or a value printed
on the pages.  ``test_oracle_pins.py`` runs them against the real oracle and
``test_oracle_mutants.py`` runs them against copies of the oracle with planted
mistakes, each of which must fail at least one pin.

Sources of the statements:
  * "State Space Models: Mamba и альтернатива Transformer" (johe.ru), S4
    section, step 3 "Convolution form": a time-invariant SSM is a causal
    convolution y = K * u with K = [C B, C A B, C A^2 B, ...] (the discrete
    B-bar is meant), and the "Параллельная форма" passage: the state is a
    sum over inputs of products of the transitions between them.
  * "Модуль 8. Альтернативы Transformer" (vladkulikov.com), section 7: the
    coefficient of input j in output i >= j is C_i^T B_j times the product of
    the transitions r = j+1..i (semi-separable matrix); the affine-pair
    operator and its worked example (tests/golden/affine_pair.txt); section
    3 "Фильтр": with stable diagonal dynamics each coordinate decays on its
    own; section 4: a NaN spreads to all later steps.
  * "Mamba и State Space Models" (nareshka.ru), "Ключевая инновация": the
    selective recurrence and the readout after the update; "Реализация
    MambaBlock": the block's depthwise Conv1d with padding d_conv - 1, cut to
    the sequence length (a causal filter), which johe.ru's MambaBlock follows
    with SiLU; vladkulikov.com sections 6 and 14: the decode cache keeps the
    last d_conv inputs of that branch and the SSM state, so a sequence can be
    continued from both.
  * The pages give no gradients; the backward is pinned to the forward by
    central finite differences.
  * Mamba-2 ("Mamba и State Space Models", "Mamba-2: State Space Duality";
    "Модуль 8", section 7): with a scalar transition per head, one operator
    has three forms, the recurrence, the semi-separable matrix
    M_ij = C_i^T B_j prod_{r=j+1..i} a_r, and the chunked matrix form that
    works inside chunks with matrix products and passes the state between
    them; with one B/C group it is the Mamba-1 scan with A and dt repeated
    over a head's channels.
  * "Модуль 8", sections 4 and 5: the exact zero-order-hold coefficient is the
    integral of e^{sA} over the step, with the limit dt at A = 0, and the
    page's worked example (tests/golden/zoh_worked_example.txt); holding the
    input constant makes the discrete state equal the continuous solution.
"""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _softplus(u):
    return np.logaddexp(0.0, u)  # log(e^0 + e^u) = log(1 + e^u), numpy's routine


def _close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    scale = max(1e-300, float(np.max(np.abs(b))))
    err = float(np.max(np.abs(a - b))) / scale
    assert err <= rtol, f"{what}: relative error {err:.3e} > {rtol:.1e}"


def _rand_case(rng, batch, L, Dn, N, dmin=-4.0, dmax=0.5):
    return dict(
        x=rng.standard_normal((batch, L, Dn)),
        delta=rng.uniform(dmin, dmax, (batch, L, Dn)),
        z=rng.standard_normal((batch, L, Dn)),
        B=rng.standard_normal((batch, L, N)),
        C=rng.standard_normal((batch, L, N)),
        A=-np.exp(rng.uniform(-1.0, 1.5, (Dn, N))),
        D=rng.standard_normal(Dn),
        delta_bias=rng.uniform(-1.0, 1.0, Dn),
    )


# --------------------------------------------------------------------------- pins


def pin_affine_worked_example(orc):
    """The pages' worked example of the affine-pair operator, exact in integers."""
    rows = np.loadtxt(os.path.join(GOLDEN, "affine_pair.txt"), comments="#", ndmin=2)
    for la, lb, ea, eb, ca, cb in rows:
        a, b = orc.affine_compose((la, lb), (ea, eb))
        assert (a[0], b[0]) == (ca, cb), f"({la},{lb}) o ({ea},{eb}) gave ({a[0]},{b[0]}), expected ({ca},{cb})"


def pin_step_size(orc):
    """softplus(delta + bias) against numpy's logaddexp(0, u); the identity branch exactly."""
    rng = np.random.default_rng(5)
    delta = np.concatenate([np.linspace(-60, 60, 241), rng.uniform(-10, 10, 259)]).reshape(5, 100)
    bias = rng.uniform(-2, 2, 100)
    got = orc.step_size(delta, bias, softplus=True)
    want = _softplus(delta + bias)
    rel = np.max(np.abs(got - want) / np.abs(want))
    assert rel < 4e-16 * 8, f"softplus relative error {rel:.2e}"
    mid = delta[np.abs(delta + bias) < 30]
    midb = np.broadcast_to(bias, delta.shape)[np.abs(delta + bias) < 30]
    textbook = np.array([math.log1p(math.exp(u)) for u in (mid + midb)])
    got_mid = got[np.abs(delta + bias) < 30]
    assert np.max(np.abs(got_mid - textbook) / textbook) < 1e-15, "softplus vs log1p(exp(u))"
    got0 = orc.step_size(delta, bias, softplus=False)
    assert np.array_equal(got0, delta + bias), "softplus=0 must give delta + bias exactly"
    # large arguments: softplus(u) -> u, tiny: softplus(u) -> e^u
    big = orc.step_size(np.array([[700.0]]), None, softplus=True)[0, 0]
    assert big == 700.0
    tiny = orc.step_size(np.array([[-700.0]]), None, softplus=True)[0, 0]
    assert abs(tiny - math.exp(-700.0)) <= 1e-15 * math.exp(-700.0)


def pin_lti_convolution(orc):
    """Time-invariant Delta, B, C: the scan equals the causal convolution y = K * x
    (+ D x, then the gate) with K_k = sum_n C_n exp(k dt A_n) dt B_n, brute force."""
    rng = np.random.default_rng(11)
    batch, L, Dn, N = 2, 40, 3, 4
    A = -np.exp(rng.uniform(-1.0, 1.5, (Dn, N)))
    Bc = rng.standard_normal((batch, N))
    Cc = rng.standard_normal((batch, N))
    dconst = rng.uniform(-3.0, 0.0, (batch, Dn))
    bias = rng.uniform(-1.0, 1.0, Dn)
    dt = _softplus(dconst + bias)                       # [batch, Dn]
    x = rng.standard_normal((batch, L, Dn))
    z = rng.standard_normal((batch, L, Dn))
    D = rng.standard_normal(Dn)
    delta = np.repeat(dconst[:, None, :], L, axis=1)
    B = np.repeat(Bc[:, None, :], L, axis=1)
    C = np.repeat(Cc[:, None, :], L, axis=1)
    out, last = orc.scan_fwd(x, delta, A, B, C, D, z, bias, softplus=True)
    k = np.arange(L, dtype=np.float64)
    # decay[b, d, k, n] = exp(k * dt[b,d] * A[d,n])
    decay = np.exp(k[None, None, :, None] * dt[:, :, None, None] * A[None, :, None, :])
    K = np.einsum("bn,bdkn->bdk", Cc, decay * (dt[:, :, None, None] * Bc[:, None, None, :]))
    y = np.zeros((batch, L, Dn))
    for t in range(L):
        for j in range(t + 1):
            y[:, t, :] += K[:, :, t - j] * x[:, j, :]
    y = (y + D * x) * _silu(z)
    _close(out, y, 1e-12, "LTI convolution")
    # final state: h[n] = sum_j exp((L-1-j) dt A_n) dt B_n x_j
    hs = np.zeros((batch, Dn, N))
    for j in range(L):
        hs += decay[:, :, L - 1 - j, :] * dt[:, :, None] * Bc[:, None, :] * x[:, j, :, None]
    _close(last, hs, 1e-12, "LTI final state")


def pin_semiseparable(orc):
    """Time-varying (selective) case: y_i = sum_{j<=i} sum_n C_i[n] exp(A_n * sum_{r=j+1..i} dt_r)
    dt_j B_j[n] x_j + D x_i, gated; brute force over (i, j) with the step sums taken directly."""
    for softplus in (True, False):
        rng = np.random.default_rng(21 + softplus)
        batch, L, Dn, N = 2, 24, 3, 3
        c = _rand_case(rng, batch, L, Dn, N, dmin=-4.0 if softplus else 0.01, dmax=0.5)
        if not softplus:
            c["delta_bias"] = rng.uniform(0.0, 0.2, Dn)
        out, last = orc.scan_fwd(softplus=softplus, **c)
        u = c["delta"] + c["delta_bias"]
        dt = _softplus(u) if softplus else u               # [batch, L, Dn]
        A, B, C, x = c["A"], c["B"], c["C"], c["x"]
        y = np.zeros((batch, L, Dn))
        hL = np.zeros((batch, Dn, N))
        for i in range(L):
            for j in range(i + 1):
                seg = dt[:, j + 1:i + 1, :].sum(axis=1)    # [batch, Dn]
                w = np.exp(seg[:, :, None] * A[None, :, :]) * (dt[:, j, :, None] * B[:, j, None, :])
                y[:, i, :] += np.einsum("bn,bdn->bd", C[:, i, :], w) * x[:, j, :]
                if i == L - 1:
                    hL += w * x[:, j, :, None]
        y = (y + c["D"] * x) * _silu(c["z"])
        _close(out, y, 1e-11, f"semi-separable form (softplus={softplus})")
        _close(last, hL, 1e-11, f"semi-separable final state (softplus={softplus})")


def pin_delta_zero(orc):
    """Delta = 0 with softplus off: the transition is the identity and the input term vanishes,
    so h stays 0 and y = D x exactly (times the gate); a tiny Delta moves y by O(Delta)."""
    rng = np.random.default_rng(31)
    batch, L, Dn, N = 2, 16, 5, 4
    c = _rand_case(rng, batch, L, Dn, N)
    c["delta"] = np.zeros_like(c["delta"])
    out, last = orc.scan_fwd(c["x"], c["delta"], c["A"], c["B"], c["C"], c["D"], None, None, softplus=False)
    assert np.array_equal(out, c["D"] * c["x"]), "Delta=0 must give y = D x exactly"
    assert np.array_equal(last, np.zeros_like(last)), "Delta=0 must leave the state at zero"
    out, _ = orc.scan_fwd(c["x"], c["delta"], c["A"], c["B"], c["C"], c["D"], c["z"], None, softplus=False)
    _close(out, c["D"] * c["x"] * _silu(c["z"]), 1e-15, "Delta=0 with the gate")
    eps = 1e-8
    out, _ = orc.scan_fwd(c["x"], c["delta"] + eps, c["A"], c["B"], c["C"], c["D"], None, None, softplus=False)
    dev = np.max(np.abs(out - c["D"] * c["x"]))
    bound = eps * L * N * np.max(np.abs(c["B"])) * np.max(np.abs(c["C"])) * np.max(np.abs(c["x"]))
    assert 0 < dev <= bound, f"Delta=1e-8 deviation {dev:.3e} outside (0, {bound:.3e}]"


def pin_impulse_closed_form(orc):
    """N = 1, constant dt, B = C = 1, x = unit impulse at t = 0, no D, no gate:
    y_t = dt * exp(t * dt * A).  With dt = 0.1 and A = -1, y_5 = 0.1 * e^{-0.5}."""
    L = 12
    x = np.zeros((1, L, 1))
    x[0, 0, 0] = 1.0
    out, last = orc.scan_fwd(x, np.full((1, L, 1), 0.1), np.array([[-1.0]]), np.ones((1, L, 1)),
                             np.ones((1, L, 1)), None, None, None, softplus=False)
    want = 0.1 * np.exp(-0.1 * np.arange(L))
    _close(out[0, :, 0], want, 1e-14, "impulse response")
    assert abs(out[0, 5, 0] - 0.1 * math.exp(-0.5)) <= 1e-15 * 0.1
    assert abs(last[0, 0, 0] - 0.1 * math.exp(-0.1 * (L - 1))) <= 1e-15 * 0.1


def pin_chunked_composition(orc):
    """The chunked form (affine pairs composed in time order) equals the sequential scan
    for every chunk length, including ones that do not divide L."""
    rng = np.random.default_rng(41)
    batch, L, Dn, N = 2, 29, 3, 4
    c = _rand_case(rng, batch, L, Dn, N)
    ref, ref_last = orc.scan_fwd(**c)
    for tc in (1, 2, 3, 7, L // 4, L - 1, L, L + 5):
        out, last = orc.scan_fwd(chunk=tc, **c)
        _close(out, ref, 1e-12, f"chunked output (chunk={tc})")
        _close(last, ref_last, 1e-12, f"chunked final state (chunk={tc})")


def pin_decode_equals_scan(orc):
    """L decode steps from a zero state reproduce one scan bitwise, and
    prefill(L1) followed by L2 decode steps equals scan(L1 + L2) bitwise; with
    the small-step and with the zero-order-hold input coefficient."""
    rng = np.random.default_rng(51)
    batch, L, Dn, N = 3, 17, 4, 5
    c = _rand_case(rng, batch, L, Dn, N)
    for zoh in (False, True):
        ref, ref_last = orc.scan_fwd(**c, zoh=zoh)
        state = np.zeros((batch, Dn, N))
        for t in range(L):
            y, state = orc.state_update(state, c["x"][:, t], c["delta"][:, t], c["A"], c["B"][:, t],
                                        c["C"][:, t], c["D"], c["z"][:, t], c["delta_bias"], zoh=zoh)
            assert np.array_equal(y, ref[:, t]), f"decode step {t} differs from the scan (zoh {zoh})"
        assert np.array_equal(state, ref_last), f"decode final state differs from the scan (zoh {zoh})"
        L1 = 9
        pre = {k: (v[:, :L1] if k in ("x", "delta", "z", "B", "C") else v) for k, v in c.items()}
        out1, st = orc.scan_fwd(**pre, zoh=zoh)
        assert np.array_equal(out1, ref[:, :L1])
        for t in range(L1, L):
            y, st = orc.state_update(st, c["x"][:, t], c["delta"][:, t], c["A"], c["B"][:, t], c["C"][:, t],
                                     c["D"], c["z"][:, t], c["delta_bias"], zoh=zoh)
            assert np.array_equal(y, ref[:, t]), f"continued decode step {t} differs (zoh {zoh})"
        assert np.array_equal(st, ref_last)


def pin_invariants(orc):
    """Linearity in x, causality, channel permutation, B*s with C/s, batch independence."""
    rng = np.random.default_rng(61)
    batch, L, Dn, N = 2, 20, 6, 4
    c = _rand_case(rng, batch, L, Dn, N)
    y, _ = orc.scan_fwd(**c)
    # linearity in x (Delta, B, C, z fixed)
    x2 = rng.standard_normal(c["x"].shape)
    y2, _ = orc.scan_fwd(**{**c, "x": x2})
    y12, _ = orc.scan_fwd(**{**c, "x": 2.0 * c["x"] - 3.0 * x2})
    _close(y12, 2.0 * y - 3.0 * y2, 1e-13, "linearity in x")
    # causality: changing x at t0 leaves every earlier output bitwise unchanged, changes later ones
    t0 = 11
    xp = c["x"].copy()
    xp[:, t0, :] += 1.0
    yp, _ = orc.scan_fwd(**{**c, "x": xp})
    assert np.array_equal(yp[:, :t0], y[:, :t0]), "output before t0 depends on x[t0]"
    assert np.all(yp[:, t0] != y[:, t0]), "output at t0 does not depend on x[t0]"
    # permutation of channels
    perm = rng.permutation(Dn)
    cp = dict(c)
    for k in ("x", "delta", "z"):
        cp[k] = c[k][:, :, perm]
    cp["A"], cp["D"], cp["delta_bias"] = c["A"][perm], c["D"][perm], c["delta_bias"][perm]
    yq, _ = orc.scan_fwd(**cp)
    assert np.array_equal(yq, y[:, :, perm]), "channel permutation"
    # B scaled by s and C by 1/s (powers of two: exact)
    ys, _ = orc.scan_fwd(**{**c, "B": c["B"] * 8.0, "C": c["C"] / 8.0})
    assert np.array_equal(ys, y), "B*s, C/s must leave y unchanged"
    # batch rows are independent
    for b in range(batch):
        cb = {k: (v[b:b + 1] if k in ("x", "delta", "z", "B", "C") else v) for k, v in c.items()}
        yb, _ = orc.scan_fwd(**cb)
        assert np.array_equal(yb[0], y[b]), f"batch row {b} depends on other rows"


def pin_decay(orc):
    """Stable diagonal dynamics (A < 0, dt > 0) with no input: every state coordinate's
    magnitude is non-increasing, step by step, and strictly decreases when nonzero."""
    rng = np.random.default_rng(71)
    batch, Dn, N = 2, 3, 4
    A = -np.exp(rng.uniform(-1.0, 1.5, (Dn, N)))
    state = rng.standard_normal((batch, Dn, N))
    zeros = np.zeros((batch, Dn))
    for t in range(10):
        delta = rng.uniform(-3, 1, (batch, Dn))
        y, nxt = orc.state_update(state, zeros, delta, A, rng.standard_normal((batch, N)),
                                  rng.standard_normal((batch, N)), None, None, None)
        assert np.all(np.abs(nxt) < np.abs(state)), f"step {t}: a coordinate did not decay"
        state = nxt


def pin_nan_propagation(orc):
    """A NaN is never dropped: in x[b,t0,d0] it reaches y[b, t>=t0, d0] and the final state of
    (b, d0) only; in B[b,t0,:] every channel of row b from t0 on; in C[b,t0,:] only step t0 of row b."""
    rng = np.random.default_rng(81)
    batch, L, Dn, N = 2, 12, 3, 4
    c = _rand_case(rng, batch, L, Dn, N)
    t0, b0, d0 = 5, 1, 2
    cx = {**c, "x": c["x"].copy()}
    cx["x"][b0, t0, d0] = np.nan
    y, last = orc.scan_fwd(**cx)
    mask = np.zeros(y.shape, bool)
    mask[b0, t0:, d0] = True
    assert np.all(np.isnan(y[mask])) and np.all(np.isfinite(y[~mask])), "NaN in x: wrong spread"
    lm = np.zeros(last.shape, bool)
    lm[b0, d0, :] = True
    assert np.all(np.isnan(last[lm])) and np.all(np.isfinite(last[~lm])), "NaN in x: wrong final state"
    cb = {**c, "B": c["B"].copy()}
    cb["B"][b0, t0, 1] = np.nan
    y, _ = orc.scan_fwd(**cb)
    mask = np.zeros(y.shape, bool)
    mask[b0, t0:, :] = True
    assert np.all(np.isnan(y[mask])) and np.all(np.isfinite(y[~mask])), "NaN in B: wrong spread"
    cc = {**c, "C": c["C"].copy()}
    cc["C"][b0, t0, 1] = np.nan
    y, _ = orc.scan_fwd(**cc)
    mask = np.zeros(y.shape, bool)
    mask[b0, t0, :] = True
    assert np.all(np.isnan(y[mask])) and np.all(np.isfinite(y[~mask])), "NaN in C: wrong spread"


def pin_optional_inputs(orc):
    """Each optional input switches exactly its own term: no D means no skip (y = C h),
    no gate means no SiLU factor, no bias means dt = softplus(delta)."""
    rng = np.random.default_rng(91)
    batch, L, Dn, N = 1, 10, 3, 4
    c = _rand_case(rng, batch, L, Dn, N)
    full, _ = orc.scan_fwd(**c)
    noD, _ = orc.scan_fwd(**{**c, "D": None})
    _close((noD / _silu(c["z"]) + c["D"] * c["x"]) * _silu(c["z"]), full, 1e-13, "D skip term")
    nogate, _ = orc.scan_fwd(**{**c, "z": None})
    _close(nogate * _silu(c["z"]), full, 1e-13, "SiLU gate factor")
    nobias, _ = orc.scan_fwd(**{**c, "delta_bias": None, "delta": c["delta"] + c["delta_bias"]})
    _close(nobias, full, 1e-13, "bias folded into delta")


def pin_initial_state_free_response(orc):
    """From a stored state h0 with no input (x = 0) the output is the state's free
    decay read out: y_t = (sum_n C_t[n] exp(A_n sum_{s<=t} dt_s) h0[n]) * SiLU(z_t),
    a closed form with cumulative step sums (no recurrence)."""
    rng = np.random.default_rng(41)
    batch, L, Dn, N = 2, 23, 3, 5
    c = _rand_case(rng, batch, L, Dn, N)
    c["x"] = np.zeros_like(c["x"])
    h0 = rng.standard_normal((batch, Dn, N))
    dt = _softplus(c["delta"] + c["delta_bias"][None, None, :])   # [b, t, d]
    S = np.cumsum(dt, axis=1)
    ref = np.einsum("btn,btdn,bdn->btd", c["C"], np.exp(S[..., None] * c["A"][None, None]), h0)
    ref = ref * _silu(c["z"])
    for chunk in (0, 5):
        out, last = orc.scan_fwd(**c, h0=h0, chunk=chunk)
        _close(out, ref, 1e-12, f"free response from h0 (chunk {chunk})")
        _close(last, np.exp(S[:, -1, :, None] * c["A"][None]) * h0, 1e-12, "final state of the free response")


def pin_initial_state_continuation(orc):
    """Scanning L1 steps, then L2 more from the stored state, is one scan of L1 + L2
    steps (bitwise: the same arithmetic in the same order); the chunked form from
    h0 agrees with the sequential one."""
    rng = np.random.default_rng(43)
    batch, L1, L2, Dn, N = 2, 9, 14, 3, 4
    c = _rand_case(rng, batch, L1 + L2, Dn, N)
    full, full_last = orc.scan_fwd(**c)
    first = {k: (v[:, :L1] if k in ("x", "delta", "z", "B", "C") else v) for k, v in c.items()}
    second = {k: (v[:, L1:] if k in ("x", "delta", "z", "B", "C") else v) for k, v in c.items()}
    o1, h1 = orc.scan_fwd(**first)
    o2, h2 = orc.scan_fwd(**second, h0=h1)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), full), "continuation differs from one scan"
    assert np.array_equal(h2, full_last), "continued final state differs"
    o2c, h2c = orc.scan_fwd(**second, h0=h1, chunk=4)
    _close(o2c, o2, 1e-12, "chunked continuation")
    _close(h2c, h2, 1e-12, "chunked continuation state")
    # an empty continuation returns the stored state unchanged
    empty = {k: (v[:, :0] if k in ("x", "delta", "z", "B", "C") else v) for k, v in c.items()}
    _, h_empty = orc.scan_fwd(**empty, h0=h1)
    assert np.array_equal(h_empty, h1)


def _conv_reference(x, w, bias, silu_on, hist=None):
    """Causal depthwise convolution per channel with numpy's convolve: the filter
    reversed (Conv1d correlates), full convolution, first L outputs; optional K
    earlier inputs prepended."""
    batch, L, Dn = x.shape
    K = w.shape[1]
    out = np.empty_like(x)
    for b in range(batch):
        for d in range(Dn):
            seq = x[b, :, d] if hist is None else np.concatenate([hist[b, d, :], x[b, :, d]])
            full = np.convolve(seq, w[d, ::-1])
            lin = full[(0 if hist is None else K):][:L] + (0.0 if bias is None else bias[d])
            out[b, :, d] = _silu(lin) if silu_on else lin
    return out


def pin_conv1d_numpy(orc):
    """The convolution equals numpy's convolve with the reversed filter (Conv1d
    with padding K - 1 cut to L steps), plus bias, through SiLU; with a cache of
    earlier inputs, the same on the joined sequence."""
    rng = np.random.default_rng(47)
    batch, L, Dn, K = 2, 19, 3, 4
    x = rng.standard_normal((batch, L, Dn))
    w = rng.standard_normal((Dn, K))
    bias = rng.standard_normal(Dn)
    for silu_on in (True, False):
        out, _ = orc.conv1d_fwd(x, w, bias, silu=silu_on)
        _close(out, _conv_reference(x, w, bias, silu_on), 1e-12, f"conv1d vs numpy (silu {silu_on})")
    hist = rng.standard_normal((batch, Dn, K))
    out, _ = orc.conv1d_fwd(x, w, None, silu=True, conv_state=hist)
    _close(out, _conv_reference(x, w, None, True, hist), 1e-12, "conv1d with a cache vs numpy")


def pin_conv1d_impulse(orc):
    """A unit impulse at t0 (no bias, no activation) returns the filter reversed:
    out[t0 + j] = w[K - 1 - j] for j < K, and 0 elsewhere."""
    batch, L, Dn, K, t0 = 1, 12, 2, 4, 3
    x = np.zeros((batch, L, Dn))
    x[0, t0, :] = 1.0
    w = np.array([[1.0, 2.0, 3.0, 4.0], [-0.5, 0.25, 8.0, -2.0]])
    out, st = orc.conv1d_fwd(x, w, None, silu=False)
    ref = np.zeros_like(x)
    for j in range(K):
        ref[0, t0 + j, :] = w[:, K - 1 - j]
    assert np.array_equal(out, ref), "impulse response is not the reversed filter"
    assert np.array_equal(st, np.zeros((batch, Dn, K))), "cache after the impulse has left it"


def pin_conv1d_decode_and_continuation(orc):
    """L decode steps from a zero cache equal one prefill (bitwise), and so does a
    prefill of L1 steps continued by a prefill of L2 steps from the returned cache;
    a sequence shorter than the filter leaves a zero-padded cache."""
    rng = np.random.default_rng(53)
    batch, L1, L2, Dn, K = 2, 6, 9, 3, 4
    x = rng.standard_normal((batch, L1 + L2, Dn))
    w = rng.standard_normal((Dn, K))
    bias = rng.standard_normal(Dn)
    full, full_st = orc.conv1d_fwd(x, w, bias)
    st = np.zeros((batch, Dn, K))
    outs = []
    for t in range(L1 + L2):
        o, st = orc.conv1d_update(st, x[:, t], w, bias)
        outs.append(o)
    assert np.array_equal(np.stack(outs, axis=1), full), "decode steps differ from the prefill"
    assert np.array_equal(st, full_st), "decode cache differs from the prefill cache"
    o1, s1 = orc.conv1d_fwd(x[:, :L1], w, bias)
    o2, s2 = orc.conv1d_fwd(x[:, L1:], w, bias, conv_state=s1)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), full), "continued prefill differs"
    assert np.array_equal(s2, full_st)
    _, s_short = orc.conv1d_fwd(x[:, :2], w, bias)
    ref = np.zeros((batch, Dn, K))
    ref[:, :, K - 2:] = np.transpose(x[:, :2], (0, 2, 1))
    assert np.array_equal(s_short, ref), "short-sequence cache is not zero-padded"


def _fd_grads(orc, case, h0, g, glast, softplus, keys, eps=1e-6):
    """Central finite differences of L = sum(g * out) + sum(glast * last_state),
    computed with the forward scan only."""
    def loss(c, hh):
        out, last = orc.scan_fwd(**c, h0=hh, softplus=softplus)
        return float(np.sum(out * g) + np.sum(last * glast))
    res = {}
    for k in keys:
        base = h0 if k == "h0" else case[k]
        num = np.zeros_like(base)
        for i in np.ndindex(base.shape):
            vals = []
            for sgn in (1.0, -1.0):
                c = {kk: v.copy() for kk, v in case.items()}
                hh = None if h0 is None else h0.copy()
                tgt = hh if k == "h0" else c[k]
                tgt[i] += sgn * eps
                vals.append(loss(c, hh))
            num[i] = (vals[0] - vals[1]) / (2 * eps)
        res[k] = num
    return res


def pin_backward_finite_differences(orc):
    """Every gradient of the backward equals the central finite difference of the
    (pinned) forward scan: L = sum(dout * out) + sum(dlast * last_state), for x,
    delta, z, B, C, A, D, delta_bias and the initial state; softplus on and off,
    with and without the optional inputs."""
    rng = np.random.default_rng(59)
    batch, L, Dn, N = 2, 6, 3, 3
    names = {"x": "dx", "delta": "ddelta", "z": "dz", "B": "dB", "C": "dC", "A": "dA", "D": "dD",
             "delta_bias": "ddelta_bias", "h0": "dh0"}
    for softplus, optional in ((True, True), (False, True), (True, False)):
        c = _rand_case(rng, batch, L, Dn, N)
        if not softplus:
            c["delta"] = rng.uniform(0.01, 0.5, c["delta"].shape)
            c["delta_bias"] = rng.uniform(0.0, 0.1, Dn)
        if not optional:
            for k in ("z", "D", "delta_bias"):
                c.pop(k)
        h0 = rng.standard_normal((batch, Dn, N)) if optional else None
        g = rng.standard_normal((batch, L, Dn))
        glast = rng.standard_normal((batch, Dn, N))
        got = orc.scan_bwd(**c, softplus=softplus, h0=h0, dout=g, dlast=glast)
        keys = list(c) + (["h0"] if h0 is not None else [])
        num = _fd_grads(orc, c, h0, g, glast, softplus, keys)
        for k in keys:
            _close(got[names[k]], num[k], 1e-7, f"d{k} vs finite differences (softplus {softplus})")
        assert set(got) == {names[k] for k in keys}, "gradients of absent inputs must be absent"


def pin_zoh_worked_example(orc):
    """The pages' worked example: for a = -1, B = 1 the small-step coefficient dt
    exceeds the exact zero-order-hold one by 10 % at dt = 0.193747558.  One step
    from zero with x = 1 and C = 1 reads out the input coefficient itself."""
    rows = np.loadtxt(os.path.join(GOLDEN, "zoh_worked_example.txt"), comments="#", ndmin=2)
    for a, bv, dt, eps in rows:
        args = dict(x=np.ones((1, 1, 1)), delta=np.full((1, 1, 1), dt), A=np.array([[a]]),
                    B=np.full((1, 1, 1), bv), C=np.ones((1, 1, 1)), softplus=False)
        y_zoh, _ = orc.scan_fwd(**args, zoh=True)
        y_dt, _ = orc.scan_fwd(**args)
        assert y_dt[0, 0, 0] == dt * bv, "the small-step coefficient is dt B"
        got = y_dt[0, 0, 0] / y_zoh[0, 0, 0] - 1.0
        # dt is printed to 9 digits and d(eps)/d(dt) is about 0.53 there
        assert abs(got - eps) <= 1e-9, f"relative error of dt B against ZOH: {got!r}, page: {eps}"


def pin_zoh_held_input_is_exact(orc):
    """With x and B held constant, zero-order hold reproduces the continuous system:
    after steps dt_1..dt_t from zero the state is (e^{A S_t} - 1) / A * B x, with
    S_t the elapsed time (S_t B x where A = 0), whatever the step sizes; so merging
    pairs of steps leaves the state unchanged.  Sequential and chunked forms.  The
    small-step coefficient fails this (control)."""
    rng = np.random.default_rng(61)
    batch, L, Dn, N = 2, 36, 3, 5
    A = -np.exp(rng.uniform(-1.0, 2.5, (Dn, N)))
    A[0, 0] = 0.0
    A[1, 1] = -1e-7
    xv = rng.standard_normal((batch, Dn))
    Bv = rng.standard_normal((batch, N))
    Cv = rng.standard_normal((batch, N))
    x = np.repeat(xv[:, None, :], L, axis=1)
    B = np.repeat(Bv[:, None, :], L, axis=1)
    C = np.repeat(Cv[:, None, :], L, axis=1)
    delta = rng.uniform(0.001, 0.4, (batch, L, Dn))
    S = np.cumsum(delta, axis=1)                                    # [b, t, d]
    AS = S[..., None] * A[None, None]                               # [b, t, d, n]
    safeA = np.where(A == 0.0, 1.0, A)
    # (e^{AS} - 1) / A, by its power series S sum_k (AS)^k / (k+1)! where |AS| is small
    series = S[..., None] * sum(AS ** k / math.factorial(k + 1) for k in range(8))
    coef = np.where(np.abs(AS) < 1e-2, series, (np.exp(AS) - 1.0) / safeA[None, None])
    h_ref = coef * Bv[:, None, None, :] * xv[:, None, :, None]       # [b, t, d, n]
    y_ref = np.einsum("btdn,bn->btd", h_ref, Cv)
    for chunk in (0, 5):
        out, last = orc.scan_fwd(x, delta, A, B, C, softplus=False, zoh=True, chunk=chunk)
        _close(out, y_ref, 1e-12, f"held-input outputs (chunk {chunk})")
        _close(last, h_ref[:, -1], 1e-12, f"held-input final state (chunk {chunk})")
    merged = delta[:, 0::2] + delta[:, 1::2]
    _, last2 = orc.scan_fwd(x[:, : L // 2], merged, A, B[:, : L // 2], C[:, : L // 2], softplus=False, zoh=True)
    _close(last2, h_ref[:, -1], 1e-12, "state after merged steps")
    _, last_dt = orc.scan_fwd(x, delta, A, B, C, softplus=False)
    assert float(np.max(np.abs(last_dt - h_ref[:, -1]))) > 1e-3 * float(np.max(np.abs(h_ref[:, -1]))), \
        "control: the small-step form is not exact for a held input"


def pin_zoh_integral_definition(orc):
    """One step's coefficient is the integral of e^{sA} over s in [0, dt]: against
    composite Simpson quadrature at several (dt, A), up to |dt A| = 40; at A = 0 it
    is dt exactly (the same as the small-step form) and it is continuous there."""
    dts = np.array([1e-3, 0.05, 0.3, 1.0, 4.0])
    A = np.array([[-10.0, -1.0, -0.25, -3e-4, 0.0, -1e-12, 0.5]])
    batch, N = dts.size, A.shape[1]
    args = dict(x=np.ones((batch, 1, 1)), delta=dts.reshape(batch, 1, 1), A=A,
                B=np.ones((batch, 1, N)), C=np.zeros((batch, 1, N)), softplus=False)
    _, h = orc.scan_fwd(**args, zoh=True)
    _, h_dt = orc.scan_fwd(**args)
    m = 20000                                                      # Simpson panels (even)
    for i, dt in enumerate(dts):
        s = np.linspace(0.0, dt, m + 1)
        w = np.ones(m + 1)
        w[1:-1:2], w[2:-1:2] = 4.0, 2.0
        for n in range(N):
            quad = float(np.sum(w * np.exp(s * A[0, n]))) * dt / (3.0 * m)
            assert abs(h[i, 0, n] - quad) <= 1e-10 * quad, f"dt={dt} A={A[0, n]}: {h[i, 0, n]!r} vs {quad!r}"
        assert h[i, 0, 4] == h_dt[i, 0, 4] == dt, "A = 0: the coefficient is dt"
        assert abs(h[i, 0, 5] - dt) <= 1e-11 * dt, "continuity at A -> 0"


def _ssd_case(rng, batch, L, H, P, G, N):
    return dict(
        x=rng.standard_normal((batch, L, H, P)),
        dt=rng.uniform(-4.0, 0.5, (batch, L, H)),
        A=-np.exp(rng.uniform(-1.0, 1.5, H)),
        B=rng.standard_normal((batch, L, G, N)),
        C=rng.standard_normal((batch, L, G, N)),
        D=rng.standard_normal(H * P),
        z=rng.standard_normal((batch, L, H, P)),
        dt_bias=rng.uniform(-1.0, 1.0, H),
    )


def pin_ssd_semiseparable(orc):
    """The Mamba-2 scan is multiplication by the semi-separable matrix
    M_ij = C_i^T B_j prod_{r=j+1..i} a_r (a_r = exp(dt_r A_h)) applied to dt x, plus
    the initial state's decay C_i^T prod_{r<=i} a_r h0, the D skip and the gate:
    brute force over (i, j) with numpy, per batch row and head, groups included."""
    rng = np.random.default_rng(71)
    batch, L, H, P, G, N = 2, 9, 4, 3, 2, 5
    c = _ssd_case(rng, batch, L, H, P, G, N)
    h0 = rng.standard_normal((batch, H, P, N))
    dt = _softplus(c["dt"] + c["dt_bias"][None, None, :])          # [b, t, h]
    ref = np.zeros((batch, L, H, P))
    ref_last = np.zeros((batch, H, P, N))
    for b in range(batch):
        for h in range(H):
            g = h // (H // G)
            a = np.exp(dt[b, :, h] * c["A"][h])
            Bm, Cm = c["B"][b, :, g], c["C"][b, :, g]                # [L, N]
            M = np.zeros((L, L))
            for i in range(L):
                for j in range(i + 1):
                    M[i, j] = (Cm[i] @ Bm[j]) * np.prod(a[j + 1:i + 1])
            u = dt[b, :, h, None] * c["x"][b, :, h]                   # [L, P]
            decay0 = np.array([np.prod(a[:i + 1]) for i in range(L)])
            y = M @ u + decay0[:, None] * (Cm @ h0[b, h].T)
            y = y + c["D"][h * P:(h + 1) * P][None, :] * c["x"][b, :, h]
            ref[b, :, h] = y * _silu(c["z"][b, :, h])
            # final state: sum_j prod_{r>j} a_r dt_j x_j B_j^T, plus the decayed h0
            w = np.array([np.prod(a[j + 1:]) for j in range(L)])
            ref_last[b, h] = (u * w[:, None]).T @ Bm + np.prod(a) * h0[b, h]
    out, last = orc.ssd_fwd(**c, h0=h0)
    _close(out, ref, 1e-12, "SSD against the semi-separable matrix")
    _close(last, ref_last, 1e-12, "SSD final state")


def _ssd_chunked(c, h0, Q):
    """The chunked matrix form in numpy: inside a chunk, Y = (L o C B^T) (dt x) with
    L_ij = exp(s_i - s_j) for j <= i (s = cumulative dt A within the chunk), plus the
    incoming state read out with decay exp(s_i); the state passed to the next chunk
    is exp(s_end) state + sum_j exp(s_end - s_j) dt_j x_j B_j^T."""
    batch, L, H, P = c["x"].shape
    G = c["B"].shape[2]
    dt = _softplus(c["dt"] + c["dt_bias"][None, None, :])
    out = np.zeros((batch, L, H, P))
    last = np.zeros_like(h0)
    for b in range(batch):
        for h in range(H):
            g = h // (H // G)
            S = h0[b, h].copy()                                      # [P, N]
            for t0 in range(0, L, Q):
                t1 = min(t0 + Q, L)
                d = dt[b, t0:t1, h]
                s = np.cumsum(d * c["A"][h])
                Bm, Cm = c["B"][b, t0:t1, g], c["C"][b, t0:t1, g]
                X = c["x"][b, t0:t1, h]
                Lm = np.tril(np.exp(s[:, None] - s[None, :]))
                y = (Lm * (Cm @ Bm.T)) @ (d[:, None] * X) + np.exp(s)[:, None] * (Cm @ S.T)
                S = np.exp(s[-1]) * S + (np.exp(s[-1] - s)[:, None] * d[:, None] * X).T @ Bm
                y = y + c["D"][h * P:(h + 1) * P][None, :] * X
                out[b, t0:t1, h] = y * _silu(c["z"][b, t0:t1, h])
            last[b, h] = S
    return out, last


def pin_ssd_chunked_matrix_form(orc):
    """The chunked matrix form (matrix products inside chunks, the state passed
    between them) equals the recurrence for chunk lengths that do and do not
    divide L."""
    rng = np.random.default_rng(73)
    batch, L, H, P, G, N = 2, 13, 4, 3, 1, 6
    c = _ssd_case(rng, batch, L, H, P, G, N)
    h0 = rng.standard_normal((batch, H, P, N))
    out, last = orc.ssd_fwd(**c, h0=h0)
    for Q in (1, 3, 4, L, L + 2):
        ref, ref_last = _ssd_chunked(c, h0, Q)
        _close(out, ref, 1e-12, f"chunked form Q={Q}")
        _close(last, ref_last, 1e-12, f"chunked form state Q={Q}")


def pin_ssd_is_mamba1_with_shared_parameters(orc):
    """With one B/C group, the Mamba-2 scan is the Mamba-1 scan over heads x headdim
    channels with A[d, n] = A[head] and the head's dt on every channel, bitwise."""
    rng = np.random.default_rng(75)
    batch, L, H, P, N = 2, 11, 3, 4, 5
    c = _ssd_case(rng, batch, L, H, P, 1, N)
    h0 = rng.standard_normal((batch, H, P, N))
    out, last = orc.ssd_fwd(**c, h0=h0)
    Dn = H * P
    ref, ref_last = orc.scan_fwd(
        c["x"].reshape(batch, L, Dn), np.repeat(c["dt"], P, axis=2), np.repeat(c["A"], P)[:, None] * np.ones((1, N)),
        c["B"][:, :, 0], c["C"][:, :, 0], c["D"], c["z"].reshape(batch, L, Dn), np.repeat(c["dt_bias"], P),
        h0=h0.reshape(batch, Dn, N))
    assert np.array_equal(out.reshape(batch, L, Dn), ref), "SSD differs from the Mamba-1 scan"
    assert np.array_equal(last.reshape(batch, Dn, N), ref_last), "SSD final state differs"


def pin_ssd_decode_and_continuation(orc):
    """L Mamba-2 decode steps reproduce one scan bitwise, and scanning L1 steps then
    L2 from the stored state is one scan of L1 + L2 steps."""
    rng = np.random.default_rng(77)
    batch, L, H, P, G, N = 2, 10, 4, 3, 2, 5
    c = _ssd_case(rng, batch, L, H, P, G, N)
    ref, ref_last = orc.ssd_fwd(**c)
    st = np.zeros((batch, H, P, N))
    for t in range(L):
        y, st = orc.ssd_state_update(st, c["x"][:, t], c["dt"][:, t], c["A"], c["B"][:, t], c["C"][:, t], c["D"],
                                     c["z"][:, t], c["dt_bias"])
        assert np.array_equal(y, ref[:, t]), f"SSD decode step {t} differs from the scan"
    assert np.array_equal(st, ref_last)
    L1 = 4
    cut = ("x", "dt", "z", "B", "C")
    o1, h1 = orc.ssd_fwd(**{k: (v[:, :L1] if k in cut else v) for k, v in c.items()})
    o2, h2 = orc.ssd_fwd(**{k: (v[:, L1:] if k in cut else v) for k, v in c.items()}, h0=h1)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), ref)
    assert np.array_equal(h2, ref_last)


ALL_PINS = [
    pin_affine_worked_example, pin_step_size, pin_lti_convolution, pin_semiseparable, pin_delta_zero,
    pin_impulse_closed_form, pin_chunked_composition, pin_decode_equals_scan, pin_invariants,
    pin_decay, pin_nan_propagation, pin_optional_inputs, pin_initial_state_free_response,
    pin_initial_state_continuation, pin_conv1d_numpy, pin_conv1d_impulse, pin_conv1d_decode_and_continuation,
    pin_backward_finite_differences, pin_zoh_worked_example, pin_zoh_held_input_is_exact,
    pin_zoh_integral_definition, pin_ssd_semiseparable, pin_ssd_chunked_matrix_form,
    pin_ssd_is_mamba1_with_shared_parameters, pin_ssd_decode_and_continuation,
]
