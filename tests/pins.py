"""Pins of the fp64 oracle: checks against what the pages and the mathematics fix.

Every check takes a `scan` callable with the oracle's signature
(u, delta, A, B, C, D, z, delta_bias, softplus) -> (y, last_state), so the same checks
run on the oracle itself (test_oracle_pins.py) and on deliberately broken copies of it
(test_oracle_mutants.py), which must each fail at least one of them.

None of these re-types the oracle's own loop: each uses a different evaluation of the
same quantity (a closed form, a convolution, an explicit sum of products, a gated RNN,
an associative composition) or an exact invariant.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy.special import expit

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = max(float(np.sqrt(np.mean(b * b))), 1e-300)
    return float(np.max(np.abs(a - b))) / scale


def _softplus_np(x):
    return np.logaddexp(0.0, np.asarray(x, np.float64))


def _sym(v):
    if isinstance(v, str):
        return {"-ln2": -math.log(2.0), "-2ln2": -2.0 * math.log(2.0), "ln3": math.log(3.0)}[v]
    return float(v)


def _rng(seed):
    return np.random.default_rng(seed)


# --- worked examples (tests/golden/worked_examples.json) -----------------------------

def check_worked_examples(scan):
    with open(GOLDEN) as f:
        ex = json.load(f)["examples"]
    ln2, ln3 = math.log(2.0), math.log(3.0)
    for e in ex:
        L, N = len(e["u"]), e["N"]
        u = np.array(e["u"], np.float64).reshape(1, L, 1)
        dl = np.array(e["delta"], np.float64).reshape(1, L, 1)
        A = np.array([[_sym(a) for a in e["A"]]], np.float64)
        B = np.array(e["B"], np.float64).reshape(1, L, N)
        C = np.array(e["C"], np.float64).reshape(1, L, N)
        D = np.array([e["D"]], np.float64)
        z = None if e["z"] is None else np.array([_sym(v) for v in e["z"]]).reshape(1, L, 1)
        bias = None if e["delta_bias"] is None else np.array([e["delta_bias"]], np.float64)
        y, h = scan(u, dl, A, B, C, D, z, bias, e["softplus"])
        if "y" in e:
            want_y, want_h = np.array(e["y"]), np.array(e["last_state"])
        elif "y_in_units_of_ln2" in e:
            want_y = ln2 * np.array(e["y_in_units_of_ln2"])
            want_h = ln2 * np.array(e["last_state_in_units_of_ln2"])
        else:
            k = np.array(e["k"])
            want_y = ln3 * (0.75 * ln2 * k + 0.375 * np.array(e["u"]))
            want_h = None
        np.testing.assert_allclose(y.reshape(-1), want_y, rtol=e["rtol"], atol=1e-15, err_msg=e["name"])
        if want_h is not None:
            np.testing.assert_allclose(h.reshape(-1), want_h, rtol=e["rtol"], atol=1e-15, err_msg=e["name"])


# --- LTI: recurrence == convolution with K_k = sum_n C_n dA_n^k delta B_n --------------
# urworte.de "Methodische Grundlagen" (convolution form for training, recurrence for
# inference); shakilmahmud.com section 3 (dual form, FFT convolution).

def lti_inputs(seed=11, L=256, D=16, N=4):
    from selective_state_space_32_amd import inputs
    c = inputs.scan_case(1, L, D, N, "f32", a_init="s4d", bias=-1.0, delta_scale=1.0, lti=True,
                         seed=seed)
    return c


def lti_kernel(c):
    """Per-channel convolution kernel K[d, k] and the per-channel step size."""
    x = c.values("delta")[0, 0, :].astype(np.float64) + c.delta_bias.astype(np.float64)
    dt = _softplus_np(x)                                   # (D,)
    A = c.A.astype(np.float64)                              # (D, N)
    Bv = c.values("B")[0, 0, :].astype(np.float64)          # (N,)
    Cv = c.values("C")[0, 0, :].astype(np.float64)
    k = np.arange(c.L, dtype=np.float64)
    dA = np.exp(dt[:, None] * A)                            # (D, N)
    powk = np.power(dA[:, :, None], k[None, None, :])       # (D, N, L)
    K = np.einsum("n,dnk->dk", Cv * Bv, powk) * dt[:, None]
    return K


def check_lti_bruteforce(scan):
    c = lti_inputs()
    u = c.values("u").astype(np.float64)[0]                 # (L, D)
    K = lti_kernel(c)
    L = c.L
    want = np.zeros((L, c.D))
    for t in range(L):
        want[t] = np.sum(K[:, t::-1][:, : t + 1] * u[: t + 1].T, axis=1)
    want += c.Dskip.astype(np.float64)[None, :] * u
    y, _ = scan(c.values("u"), c.values("delta"), c.A, c.values("B"), c.values("C"), c.Dskip, None,
                c.delta_bias, True)
    assert _rel(y[0], want) < 1e-12, _rel(y[0], want)


def check_lti_fft(scan):
    c = lti_inputs(seed=12)
    u = c.values("u").astype(np.float64)[0]
    K = lti_kernel(c)
    L = c.L
    nfft = 2 * L
    Y = np.fft.irfft(np.fft.rfft(K, nfft, axis=1) * np.fft.rfft(u.T, nfft, axis=1), nfft, axis=1)[:, :L]
    want = Y.T + c.Dskip.astype(np.float64)[None, :] * u
    y, _ = scan(c.values("u"), c.values("delta"), c.A, c.values("B"), c.values("C"), c.Dskip, None,
                c.delta_bias, True)
    assert _rel(y[0], want) < 1e-11, _rel(y[0], want)


# --- selective (time-varying) case: explicit sum of products ----------------------------
# h_t = sum_{s<=t} exp(A * sum_{r=s+1..t} delta_r) * delta_s * B_s * u_s  (the recurrence
# unrolled; the decay is taken as one exponential of a summed step size, not as a
# product of per-step factors).

def check_product_form(scan, seed=5, bsz=2, L=48, D=3, N=3):
    rng = _rng(seed)
    u = rng.standard_normal((bsz, L, D))
    x = 0.7 * rng.standard_normal((bsz, L, D))
    bias = rng.uniform(-2.0, 0.5, D)
    A = -np.exp(rng.normal(0.5, 0.6, (D, N)))
    B = rng.standard_normal((bsz, L, N))
    C = rng.standard_normal((bsz, L, N))
    Dv = rng.standard_normal(D)
    z = rng.standard_normal((bsz, L, D))
    y, h = scan(u, x, A, B, C, Dv, z, bias, True)
    dt = _softplus_np(x + bias[None, None, :])             # (bsz, L, D)
    cs = np.cumsum(dt, axis=1)                              # S_t
    want_y = np.zeros((bsz, L, D))
    want_h = np.zeros((bsz, D, N))
    for b in range(bsz):
        for d in range(D):
            for t in range(L):
                s = np.arange(t + 1)
                decay = np.exp(A[d][None, :] * (cs[b, t, d] - cs[b, s, d])[:, None])   # (t+1, N)
                ht = np.sum(decay * (dt[b, s, d] * u[b, s, d])[:, None] * B[b, s, :], axis=0)
                yt = float(C[b, t] @ ht) + Dv[d] * u[b, t, d]
                want_y[b, t, d] = yt * z[b, t, d] * expit(z[b, t, d])
                if t == L - 1:
                    want_h[b, d] = ht
    assert _rel(y, want_y) < 1e-11, _rel(y, want_y)
    assert _rel(h, want_h) < 1e-11, _rel(h, want_h)


# --- Theorem 1 (azimuth.plus/paper/mamba, gating section): N = 1, A = -1 -----------------
# exp(-softplus(x)) = 1 - sigmoid(x); with B_t chosen as sigmoid(x_t)/softplus(x_t) the
# input coefficient is g_t = sigmoid(x_t), so the scan is the gated RNN
# h_t = (1 - g_t) h_{t-1} + g_t u_t.

def check_theorem1(scan, seed=7, L=200, D=4):
    rng = _rng(seed)
    x = 2.0 * rng.standard_normal((1, L, D))
    u = rng.standard_normal((1, L, D))
    A = -np.ones((D, 1))
    g = expit(x)
    y_all = np.zeros((1, L, D))
    for d in range(D):
        # B is one vector per token shared by channels, so run one channel at a time
        B = (g[0, :, d] / _softplus_np(x[0, :, d])).reshape(1, L, 1)
        C = np.ones((1, L, 1))
        yd, _ = scan(u[:, :, d:d + 1], x[:, :, d:d + 1], A[d:d + 1], B, C, None, None, None, True)
        y_all[0, :, d] = yd[0, :, 0]
    want = np.zeros((1, L, D))
    h = np.zeros(D)
    for t in range(L):
        h = (1.0 - g[0, t]) * h + g[0, t] * u[0, t]
        want[0, t] = h
    assert _rel(y_all, want) < 1e-13, _rel(y_all, want)


# --- gate limits (azimuth.plus/paper/mamba, selection section, the two gate bullets) ----

def _rand_case(seed, bsz=1, L=64, D=5, N=4):
    rng = _rng(seed)
    return dict(u=rng.standard_normal((bsz, L, D)), x=0.5 * rng.standard_normal((bsz, L, D)) + 0.2,
                A=-np.exp(rng.normal(1.0, 0.5, (D, N))), B=rng.standard_normal((bsz, L, N)),
                C=rng.standard_normal((bsz, L, N)), Dv=rng.standard_normal(D),
                z=rng.standard_normal((bsz, L, D)))


def check_small_delta_keeps_state(scan):
    """delta = 0 at token t (softplus off, no bias): exp(0) = 1 and the input term is 0,
    so the state is carried unchanged -- bitwise."""
    k = _rand_case(21)
    t0 = 40
    x = np.abs(k["x"])
    x[:, t0, :] = 0.0
    _, h_before = scan(k["u"][:, :t0], x[:, :t0], k["A"], k["B"][:, :t0], k["C"][:, :t0], k["Dv"], None, None, False)
    _, h_at = scan(k["u"][:, :t0 + 1], x[:, :t0 + 1], k["A"], k["B"][:, :t0 + 1], k["C"][:, :t0 + 1], k["Dv"], None, None, False)
    assert np.array_equal(h_before, h_at)
    y, _ = scan(k["u"][:, :t0 + 1], x[:, :t0 + 1], k["A"], k["B"][:, :t0 + 1], k["C"][:, :t0 + 1], k["Dv"], None, None, False)
    want = np.einsum("bdn,bn->bd", h_before, k["C"][:, t0]) + k["Dv"][None] * k["u"][:, t0]
    np.testing.assert_allclose(y[:, t0], want, rtol=1e-13, atol=1e-14)


def check_large_delta_resets_state(scan):
    """delta * A <= -1e4 at token t: exp underflows to exactly 0, the old state is
    forgotten and the state becomes delta*B_t*u_t; from t on the outputs equal those of
    the sequence restarted at t -- bitwise."""
    k = _rand_case(22)
    t0 = 30
    x = np.abs(k["x"])
    x[:, t0, :] = 1e4
    y, h = scan(k["u"], x, k["A"], k["B"], k["C"], k["Dv"], k["z"], None, False)
    y2, h2 = scan(k["u"][:, t0:], x[:, t0:], k["A"], k["B"][:, t0:], k["C"][:, t0:], k["Dv"], k["z"][:, t0:], None, False)
    assert np.array_equal(y[:, t0:], y2)
    assert np.array_equal(h, h2)


# --- linearity, causality, zero input, B = 0 / C = 0 ------------------------------------

def check_linearity(scan):
    k = _rand_case(23)
    rng = _rng(24)
    u2 = rng.standard_normal(k["u"].shape)
    a, b = 0.75, -1.5
    args = (k["x"], k["A"], k["B"], k["C"], k["Dv"], k["z"], None, True)
    y1, h1 = scan(k["u"], *args)
    y2, h2 = scan(u2, *args)
    y3, h3 = scan(a * k["u"] + b * u2, *args)
    assert _rel(y3, a * y1 + b * y2) < 1e-12
    assert _rel(h3, a * h1 + b * h2) < 1e-12


def check_causality(scan):
    k = _rand_case(25)
    t0 = 20
    u2 = k["u"].copy()
    u2[:, t0 + 1:] += 3.0
    x2 = k["x"].copy()
    x2[:, t0 + 1:] -= 1.0
    y1, _ = scan(k["u"], k["x"], k["A"], k["B"], k["C"], k["Dv"], k["z"], None, True)
    y2, _ = scan(u2, x2, k["A"], k["B"], k["C"], k["Dv"], k["z"], None, True)
    assert np.array_equal(y1[:, : t0 + 1], y2[:, : t0 + 1])
    assert not np.array_equal(y1[:, t0 + 1:], y2[:, t0 + 1:])


def check_zero_input(scan):
    k = _rand_case(26)
    y, h = scan(np.zeros_like(k["u"]), k["x"], k["A"], k["B"], k["C"], k["Dv"], k["z"], None, True)
    assert not np.any(y) and not np.any(h)


def check_b_or_c_zero(scan):
    """B = 0 (no input reaches the state) or C = 0 (nothing read out) leaves the gated
    skip term alone: y = D u silu(z), silu(z) = z * sigmoid(z)."""
    k = _rand_case(27)
    want = k["Dv"][None, None, :] * k["u"] * k["z"] * expit(k["z"])
    for Bz, Cz in ((np.zeros_like(k["B"]), k["C"]), (k["B"], np.zeros_like(k["C"]))):
        y, h = scan(k["u"], k["x"], k["A"], Bz, Cz, k["Dv"], k["z"], None, True)
        np.testing.assert_allclose(y, want, rtol=1e-14, atol=1e-15)


# --- associativity: chunk summaries composed with (a1,b1)o(a2,b2) = (a1 a2, a2 b1 + b2) --
# azimuth.plus/paper/mamba, hardware-aware algorithm section, parallel-scan bullet.

def check_chunk_composition(scan, seed=28, L=96, chunk=17):
    rng = _rng(seed)
    D, N = 3, 4
    u = rng.standard_normal((1, L, D))
    x = 0.6 * rng.standard_normal((1, L, D))
    A = -np.exp(rng.normal(0.3, 0.5, (D, N)))
    B = rng.standard_normal((1, L, N))
    C = rng.standard_normal((1, L, N))
    _, h_full = scan(u, x, A, B, C, None, None, None, True)
    carry_a = np.ones((D, N))
    carry_b = np.zeros((D, N))
    for s in range(0, L, chunk):
        e = min(L, s + chunk)
        _, hc = scan(u[:, s:e], x[:, s:e], A, B[:, s:e], C[:, s:e], None, None, None, True)
        dsum = np.sum(_softplus_np(x[0, s:e]), axis=0)         # (D,)
        a = np.exp(A * dsum[:, None])
        carry_a, carry_b = carry_a * a, a * carry_b + hc[0]
    assert _rel(h_full[0], carry_b) < 1e-12


def check_softplus_values(scan):
    """softplus through the oracle: N = 1, A = 0 (decay 1), B = C = u = 1, one token, so
    y = delta = softplus(x).  softplus(0) = ln 2; softplus(x) -> x for large x and -> e^x
    for very negative x."""
    xs = np.array([0.0, 50.0, 800.0, -40.0, -800.0, 1.5])
    want = np.array([math.log(2.0), 50.0 + math.exp(-50.0), 800.0, math.exp(-40.0), 0.0,
                     math.log1p(math.exp(1.5))])
    for x, w in zip(xs, want):
        y, _ = scan(np.ones((1, 1, 1)), np.full((1, 1, 1), x), np.zeros((1, 1)), np.ones((1, 1, 1)),
                    np.ones((1, 1, 1)), None, None, None, True)
        assert abs(y[0, 0, 0] - w) <= 1e-15 * max(1.0, abs(w)) + 1e-300, (x, y[0, 0, 0], w)


ALL_CHECKS = [
    check_worked_examples, check_lti_bruteforce, check_lti_fft, check_product_form,
    check_theorem1, check_small_delta_keeps_state, check_large_delta_resets_state,
    check_linearity, check_causality, check_zero_input, check_b_or_c_zero,
    check_chunk_composition, check_softplus_values,
]


# --- the scan continued from a given state ------------------------------------------------
# scan_from(u, x, A, B, C, D, z, bias, softplus, h0) -> (y, last_state)

def check_h0_no_input_decay(scan_from, seed=51, L=40, D=3, N=4):
    """With B = 0 nothing enters the state: it only decays, h_t = exp(A * S_t) h0 with S_t
    the running sum of step sizes, so y_t = (C_t . h_t + D u_t) silu(z_t) in closed form."""
    rng = _rng(seed)
    u = rng.standard_normal((1, L, D))
    x = 0.5 * rng.standard_normal((1, L, D))
    bias = rng.uniform(-2.0, 0.0, D)
    A = -np.exp(rng.normal(0.5, 0.5, (D, N)))
    B = np.zeros((1, L, N))
    C = rng.standard_normal((1, L, N))
    Dv = rng.standard_normal(D)
    z = rng.standard_normal((1, L, D))
    h0 = rng.standard_normal((1, D, N))
    y, h = scan_from(u, x, A, B, C, Dv, z, bias, True, h0)
    S = np.cumsum(_softplus_np(x[0] + bias), axis=0)            # (L, D)
    ht = np.exp(A[None] * S[:, :, None]) * h0[0][None]          # (L, D, N)
    yref = (np.einsum("tn,tdn->td", C[0], ht) + Dv * u[0]) * z[0] / (1.0 + np.exp(-z[0]))
    assert _rel(y[0], yref) < 1e-12
    assert _rel(h[0], ht[-1]) < 1e-12


def check_h0_composition(scan_from, seed=52, L=70, split=29, D=3, N=4):
    """Running tokens [0, s) from h0 and then [s, L) from the state reached equals one run
    over [0, L) from h0 (the state is all the recurrence carries)."""
    rng = _rng(seed)
    u = rng.standard_normal((2, L, D))
    x = 0.6 * rng.standard_normal((2, L, D))
    A = -np.exp(rng.normal(0.3, 0.5, (D, N)))
    B = rng.standard_normal((2, L, N))
    C = rng.standard_normal((2, L, N))
    Dv = rng.standard_normal(D)
    z = rng.standard_normal((2, L, D))
    h0 = rng.standard_normal((2, D, N))
    y, h = scan_from(u, x, A, B, C, Dv, z, None, True, h0)
    y1, h1 = scan_from(u[:, :split], x[:, :split], A, B[:, :split], C[:, :split], Dv, z[:, :split], None, True, h0)
    y2, h2 = scan_from(u[:, split:], x[:, split:], A, B[:, split:], C[:, split:], Dv, z[:, split:], None, True, h1)
    assert _rel(y, np.concatenate([y1, y2], axis=1)) < 1e-12
    assert _rel(h, h2) < 1e-12


def check_h0_linear_without_input(scan_from, seed=53, L=30, D=2, N=3):
    """With u = 0 (no input, no skip term) and no gate, y and the final state are linear in
    the initial state."""
    rng = _rng(seed)
    u = np.zeros((1, L, D))
    x = 0.5 * rng.standard_normal((1, L, D))
    A = -np.exp(rng.normal(0.0, 0.5, (D, N)))
    B = rng.standard_normal((1, L, N))
    C = rng.standard_normal((1, L, N))
    ha, hb = rng.standard_normal((1, D, N)), rng.standard_normal((1, D, N))
    ya, la = scan_from(u, x, A, B, C, None, None, None, True, ha)
    yb, lb = scan_from(u, x, A, B, C, None, None, None, True, hb)
    yab, lab = scan_from(u, x, A, B, C, None, None, None, True, 2.0 * ha - 3.0 * hb)
    assert _rel(yab, 2.0 * ya - 3.0 * yb) < 1e-12
    assert _rel(lab, 2.0 * la - 3.0 * lb) < 1e-12


H0_CHECKS = [check_h0_no_input_decay, check_h0_composition, check_h0_linear_without_input]


# --- the exact zero-order-hold input term ----------------------------------------------------
# scan_zoh(u, x, A, B, C, D, z, bias, softplus) -> (y, last_state), the scan with
# B_bar = (exp(delta A) - 1) / A * B (delta * B where A = 0) in place of delta * B.

def check_zoh_theorem1(scan_zoh, seed=61, L=200, D=4):
    """Theorem 1 (azimuth.plus/paper/mamba) exactly: with N = 1, A = -1, B = C = 1 and
    delta = softplus(x), the zero-order hold gives h_t = (1 - g_t) h_{t-1} + g_t u_t with
    g_t = sigmoid(x_t), the gated recurrence, evaluated here directly."""
    rng = _rng(seed)
    x = 2.0 * rng.standard_normal((1, L, D))
    u = rng.standard_normal((1, L, D))
    A = -np.ones((D, 1))
    B = np.ones((1, L, 1))
    C = np.ones((1, L, 1))
    y, last = scan_zoh(u, x, A, B, C, None, None, None, True)
    g = expit(x)
    want = np.zeros((1, L, D))
    h = np.zeros(D)
    for t in range(L):
        h = (1.0 - g[0, t]) * h + g[0, t] * u[0, t]
        want[0, t] = h
    assert _rel(y, want) < 1e-13, _rel(y, want)
    assert _rel(last[:, :, 0], want[:, -1]) < 1e-13


def check_zoh_continuous_solution(scan_zoh, seed=62, L=60, D=3, N=5):
    """Zero-order hold is exact for an input held constant: with u and B constant in time
    and any positive step sizes, the state after t steps is the solution of
    h' = A h + B u from h(0) = 0 at time S_t = sum of the step sizes,
    h_t[n] = (exp(A[n] S_t) - 1) / A[n] * B[n] * u (yapayzekasozluk.tr "Temel Matematiksel
    Cerceve": the continuous model that the discretisation samples).  A includes small
    magnitudes, where exp(A S) - 1 must not lose its digits."""
    rng = _rng(seed)
    dt = rng.uniform(1e-4, 0.3, (1, L, D))
    A = -np.exp(rng.normal(0.0, 1.5, (D, N)))
    A[0, 0] = -1e-7
    A[1, 2] = -3e-4
    Bv = rng.standard_normal(N)
    uv = rng.standard_normal(D)
    u = np.broadcast_to(uv, (1, L, D)).copy()
    B = np.broadcast_to(Bv, (1, L, N)).copy()
    C = rng.standard_normal((1, L, N))
    y, last = scan_zoh(u, dt, A, B, C, None, None, None, False)
    S = np.cumsum(dt[0], axis=0)                                      # (L, D)
    h = np.expm1(A[None] * S[:, :, None]) / A[None] * Bv[None, None] * uv[None, :, None]   # (L, D, N)
    want = np.einsum("tdn,tn->td", h, C[0])[None]
    assert _rel(y, want) < 1e-12, _rel(y, want)
    assert _rel(last[0], h[-1]) < 1e-12


def check_zoh_lti_bruteforce(scan_zoh, seed=63, L=120, D=4, N=3):
    """With delta, B and C constant the exact-ZOH scan is the convolution
    y_t = sum_k K_k u_{t-k} + D u_t with K_k = sum_n C_n exp(delta A_n)^k B_bar_n and
    B_bar_n = (exp(delta A_n) - 1) / A_n * B_n (shakilmahmud.com section 3's convolutional
    form), summed here term by term."""
    rng = _rng(seed)
    dtv = rng.uniform(0.01, 0.5, D)
    A = -np.exp(rng.normal(0.5, 0.7, (D, N)))
    Bv = rng.standard_normal(N)
    Cv = rng.standard_normal(N)
    Dv = rng.standard_normal(D)
    u = rng.standard_normal((1, L, D))
    dt = np.broadcast_to(dtv, (1, L, D)).copy()
    y, _ = scan_zoh(u, dt, A, np.broadcast_to(Bv, (1, L, N)).copy(), np.broadcast_to(Cv, (1, L, N)).copy(),
                    Dv, None, None, False)
    want = np.zeros((1, L, D))
    for d in range(D):
        a = np.exp(dtv[d] * A[d])
        bbar = np.expm1(dtv[d] * A[d]) / A[d] * Bv
        K = np.array([np.sum(Cv * a ** k * bbar) for k in range(L)])
        for t in range(L):
            want[0, t, d] = np.sum(K[:t + 1][::-1] * u[0, :t + 1, d]) + Dv[d] * u[0, t, d]
    assert _rel(y, want) < 1e-12, _rel(y, want)


def check_zoh_zero_A(scan_zoh, seed=64, L=50, D=2, N=3):
    """Where A = 0 nothing decays and B_bar = delta B (the limit of (exp(delta A) - 1) / A):
    the state is the running sum of delta_t B_t u_t, evaluated here with a cumulative sum."""
    rng = _rng(seed)
    dt = rng.uniform(0.01, 1.0, (1, L, D))
    u = rng.standard_normal((1, L, D))
    B = rng.standard_normal((1, L, N))
    C = rng.standard_normal((1, L, N))
    A = np.zeros((D, N))
    y, last = scan_zoh(u, dt, A, B, C, None, None, None, False)
    h = np.cumsum(dt[0, :, :, None] * u[0, :, :, None] * B[0, :, None, :], axis=0)   # (L, D, N)
    assert _rel(y[0], np.einsum("tdn,tn->td", h, C[0])) < 1e-12
    assert _rel(last[0], h[-1]) < 1e-12


ZOH_CHECKS = [check_zoh_theorem1, check_zoh_continuous_solution, check_zoh_lti_bruteforce, check_zoh_zero_A]


# --- the causal depthwise convolution and SiLU of the block's main branch ---------------------
# conv(x, w, bias, state, silu) -> (out, state_out)
# (azimuth.plus/paper/mamba, block architecture section: a short 1-D convolution of kernel
# size 4, then SiLU, produce the scan's input)

def _conv_case(seed, bsz=2, L=37, D=5, width=4):
    rng = _rng(seed)
    return (rng.standard_normal((bsz, L, D)), rng.standard_normal((D, width)), rng.standard_normal(D), rng)


def check_conv_numpy_convolve(conv, seed=81):
    """Without SiLU and from a zero history, each channel is numpy's full convolution of
    its inputs with its reversed filter, cut to the first L outputs, plus the bias."""
    for width in (1, 2, 3, 4):
        x, w, bias, _ = _conv_case(seed + width, width=width)
        out, _ = conv(x, w, bias, None, False)
        want = np.empty_like(x)
        for b in range(x.shape[0]):
            for d in range(x.shape[2]):
                want[b, :, d] = np.convolve(x[b, :, d], w[d, ::-1])[:x.shape[1]] + bias[d]
        assert _rel(out, want) < 1e-14, (width, _rel(out, want))


def check_conv_impulse(conv, seed=82, L=20, D=3, width=4):
    """A unit impulse at token t0 gives the filter back, newest tap first: out[t0 + j] =
    bias + w[width - 1 - j] for j < width, and the bias alone elsewhere (causal)."""
    rng = _rng(seed)
    w = rng.standard_normal((D, width))
    bias = rng.standard_normal(D)
    t0 = 7
    x = np.zeros((1, L, D))
    x[0, t0] = 1.0
    out, _ = conv(x, w, bias, None, False)
    for t in range(L):
        j = t - t0
        want = bias + (w[:, width - 1 - j] if 0 <= j < width else 0.0)
        assert np.all(out[0, t] == want), (t, out[0, t], want)


def check_conv_silu(conv, seed=83):
    """With SiLU the output is v * sigmoid(v) of the pre-activation (scipy's expit)."""
    x, w, bias, _ = _conv_case(seed)
    pre, _ = conv(x, w, bias, None, False)
    out, _ = conv(x, w, bias, None, True)
    assert _rel(out, pre * expit(pre)) < 1e-14


def check_conv_continuation(conv, seed=84):
    """Running the inputs in two pieces, the second from the first's state, is bitwise the
    run over the whole; the state is the last width-1 inputs (oldest first), also when a
    piece is shorter than the history."""
    for width in (2, 4):
        x, w, bias, rng = _conv_case(seed + width, L=41, width=width)
        st0 = rng.standard_normal((x.shape[0], width - 1, x.shape[2]))
        whole, st_whole = conv(x, w, bias, st0, True)
        for cut in (1, 2, 17, 40):
            a, sa = conv(x[:, :cut], w, bias, st0, True)
            bb, sb = conv(x[:, cut:], w, bias, sa, True)
            assert np.array_equal(np.concatenate([a, bb], axis=1), whole), (width, cut)
            assert np.array_equal(sb, st_whole)
        assert np.array_equal(st_whole, x[:, -(width - 1):])
        hist = np.concatenate([st0, x[:, :1]], axis=1)
        _, s1 = conv(x[:, :1], w, bias, st0, True)
        assert np.array_equal(s1, hist[:, -(width - 1):])


def check_conv_state_is_history(conv, seed=85):
    """A state equals inputs before token 0: the run from a state gives the tail of the run
    over (state rows, x) from a zero history."""
    x, w, bias, rng = _conv_case(seed, L=30)
    st0 = rng.standard_normal((x.shape[0], 3, x.shape[2]))
    out, _ = conv(x, w, bias, st0, False)
    full, _ = conv(np.concatenate([st0, x], axis=1), w, bias, None, False)
    assert _rel(out, full[:, 3:]) < 1e-15


CONV_CHECKS = [check_conv_numpy_convolve, check_conv_impulse, check_conv_silu, check_conv_continuation,
               check_conv_state_is_history]


# --- gradients of the convolution -----------------------------------------------------------
# conv_bwd(x, w, dout, bias, state, silu) -> dict dx, dw (+ dbias, dstate when given)

def _check_conv_bwd_fd(conv, conv_bwd, seed, width, silu, L=11):
    """Every gradient against a central difference of the forward (fp64, eps = 1e-6) along a
    random direction; the loss is sum(dout * out)."""
    x, w, bias, rng = _conv_case(seed, L=L, D=3, width=width)
    state = rng.standard_normal((x.shape[0], width - 1, x.shape[2]))
    dout = rng.standard_normal(x.shape)
    g = conv_bwd(x, w, dout, bias, state, silu)
    c = dict(x=x, w=w, bias=bias, state=state)

    def loss(**kw):
        a = dict(c)
        a.update(kw)
        out, _ = conv(a["x"], a["w"], a["bias"], a["state"], silu)
        return float(np.sum(dout * out))

    eps = 1e-6
    for name, gk in (("x", "dx"), ("w", "dw"), ("bias", "dbias"), ("state", "dstate")):
        if width == 1 and name == "state":
            continue
        V = rng.standard_normal(np.shape(c[name]))
        fd = (loss(**{name: c[name] + eps * V}) - loss(**{name: c[name] - eps * V})) / (2 * eps)
        an = float(np.sum(g[gk] * V))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (width, silu, name, fd, an)


def check_conv_bwd_fd_silu(conv, conv_bwd):
    for width in (2, 4):
        _check_conv_bwd_fd(conv, conv_bwd, 86 + width, width, True)


def check_conv_bwd_fd_linear(conv, conv_bwd):
    for width in (1, 3):
        _check_conv_bwd_fd(conv, conv_bwd, 90 + width, width, False, L=2)


def check_conv_bwd_adjoint(conv, conv_bwd, seed=95):
    """Without SiLU and bias the convolution is linear in (state, x) and in w separately, so
    the backward is its transpose exactly: sum(dout * out) = sum(dx * x) + sum(dstate * state)
    = sum(dw * w); and dbias = the sum of dout over sequences and tokens (pre = out)."""
    x, w, bias, rng = _conv_case(seed, L=23, D=4, width=4)
    state = rng.standard_normal((x.shape[0], 3, x.shape[2]))
    dout = rng.standard_normal(x.shape)
    out, _ = conv(x, w, None, state, False)
    g = conv_bwd(x, w, dout, bias, state, False)
    lhs = float(np.sum(dout * out))
    assert abs(float(np.sum(g["dx"] * x) + np.sum(g["dstate"] * state)) - lhs) <= 1e-12 * max(1.0, abs(lhs))
    assert abs(float(np.sum(g["dw"] * w)) - lhs) <= 1e-12 * max(1.0, abs(lhs))
    assert _rel(g["dbias"], np.sum(dout, axis=(0, 1))) < 1e-14


def check_conv_bwd_width1(conv, conv_bwd, seed=96):
    """Width 1 is a per-element map out = silu(w x + b): dx = dout silu'(p) w,
    dw = sum dout silu'(p) x, dbias = sum dout silu'(p), with silu'(p) = s + p s (1 - s),
    s = expit(p) (scipy)."""
    x, w, bias, rng = _conv_case(seed, L=17, D=4, width=1)
    dout = rng.standard_normal(x.shape)
    p = w[:, 0] * x + bias
    s = expit(p)
    gp = dout * (s + p * s * (1.0 - s))
    g = conv_bwd(x, w, dout, bias, None, True)
    assert _rel(g["dx"], gp * w[:, 0]) < 1e-13
    assert _rel(g["dw"][:, 0], np.sum(gp * x, axis=(0, 1))) < 1e-13
    assert _rel(g["dbias"], np.sum(gp, axis=(0, 1))) < 1e-13


def check_conv_bwd_causal(conv, conv_bwd, seed=97, t0=9):
    """Causality seen from the backward: a loss on out[t0] alone reaches only the inputs
    t0 - width + 1 .. t0 (dx is zero after t0 and before t0 - width + 1), with the filter
    taps in order: dx[t0 - (width-1) + k] = w[k] g[t0]."""
    x, w, bias, rng = _conv_case(seed, L=20, D=3, width=4)
    dout = np.zeros_like(x)
    dout[:, t0] = rng.standard_normal((x.shape[0], x.shape[2]))
    g = conv_bwd(x, w, dout, bias, None, False)
    assert np.all(g["dx"][:, t0 + 1:] == 0.0) and np.all(g["dx"][:, : t0 - 3] == 0.0)
    for k in range(4):
        assert _rel(g["dx"][:, t0 - 3 + k], w[:, k] * dout[:, t0]) < 1e-15


CONV_BWD_CHECKS = [check_conv_bwd_fd_silu, check_conv_bwd_fd_linear, check_conv_bwd_adjoint,
                   check_conv_bwd_width1, check_conv_bwd_causal]


# --- Mamba-2's state space dual layer (SSD) -------------------------------------------------
# ssd(x, dt, A, B, C, D, z, dt_bias, softplus, h0) -> (y, last_state)
# x, z: (b, L, H, P); dt: (b, L, H); A, D, dt_bias: (H,); B, C: (b, L, G, N); h0: (b, H, P, N)

def _ssd_case(seed, b=2, L=29, H=4, P=3, G=2, N=5, full=True):
    rng = _rng(seed)
    c = dict(x=rng.standard_normal((b, L, H, P)), dt=0.5 * rng.standard_normal((b, L, H)),
             A=-np.exp(rng.normal(0.0, 0.7, H)), B=rng.standard_normal((b, L, G, N)),
             C=rng.standard_normal((b, L, G, N)), D=None, z=None, dt_bias=None, h0=None)
    if full:
        c.update(D=rng.standard_normal(H), z=rng.standard_normal((b, L, H, P)), dt_bias=rng.uniform(-1.5, 0.0, H),
                 h0=rng.standard_normal((b, H, P, N)))
    return c


def _run_ssd(ssd, c, softplus=True):
    return ssd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["z"], c["dt_bias"], softplus, c["h0"])


def check_ssd_is_broadcast_scan(ssd, scan_from, seed=91):
    """A head is the selective scan of its P channels with the head's A in every state, the
    head's step size on every channel and its group's B and C (mugbit.ir: Mamba-2 keeps the
    SSM and makes the state matrix a scalar per head); run through the pinned scan oracle."""
    c = _ssd_case(seed)
    y, last = _run_ssd(ssd, c)
    b, L, H, P = c["x"].shape
    G, N = c["B"].shape[2], c["B"].shape[3]
    hpg = H // G
    for g in range(G):
        hs = list(range(g * hpg, (g + 1) * hpg))
        u = c["x"][:, :, hs, :].reshape(b, L, hpg * P)
        delta = np.repeat(c["dt"][:, :, hs], P, axis=2)
        A = np.repeat(c["A"][hs], P)[:, None] * np.ones((1, N))
        Dv = np.repeat(c["D"][hs], P)
        z = c["z"][:, :, hs, :].reshape(b, L, hpg * P)
        bias = np.repeat(c["dt_bias"][hs], P)
        h0 = c["h0"][:, hs].reshape(b, hpg * P, N)
        ys, ls = scan_from(u, delta, A, c["B"][:, :, g], c["C"][:, :, g], Dv, z, bias, True, h0)
        assert _rel(y[:, :, hs, :].reshape(b, L, hpg * P), ys) < 1e-13, g
        assert _rel(last[:, hs].reshape(b, hpg * P, N), ls) < 1e-13, g


def check_ssd_semiseparable(ssd, seed=92):
    """The dual form: the layer is y = M (dt x) + D x with the 1-semiseparable matrix
    M[t, s] = (C_t . B_s) exp(A (S_t - S_s)) for s <= t, 0 above the diagonal, S the running
    sum of step sizes (mugbit.ir, structured state space duality), built here as an L x L
    matrix per head and applied with numpy."""
    c = _ssd_case(seed)
    c["h0"] = None
    c["z"] = None
    y, _ = _run_ssd(ssd, c, softplus=True)
    b, L, H, P = c["x"].shape
    hpg = H // c["B"].shape[2]
    want = np.zeros_like(y)
    for bb in range(b):
        for h in range(H):
            g = h // hpg
            dt = _softplus_np(c["dt"][bb, :, h] + c["dt_bias"][h])
            S = np.cumsum(dt)
            M = (c["C"][bb, :, g] @ c["B"][bb, :, g].T) * np.tril(np.exp(c["A"][h] * (S[:, None] - S[None, :])))
            want[bb, :, h] = M @ (dt[:, None] * c["x"][bb, :, h]) + c["D"][h] * c["x"][bb, :, h]
    assert _rel(y, want) < 1e-12, _rel(y, want)


def check_ssd_composition(ssd, seed=93, split=11):
    """Two pieces, the second from the first's state, are bitwise the run over the whole."""
    c = _ssd_case(seed)
    y, last = _run_ssd(ssd, c)
    c1 = dict(c, x=c["x"][:, :split], dt=c["dt"][:, :split], B=c["B"][:, :split], C=c["C"][:, :split],
              z=c["z"][:, :split])
    y1, l1 = _run_ssd(ssd, c1)
    c2 = dict(c, x=c["x"][:, split:], dt=c["dt"][:, split:], B=c["B"][:, split:], C=c["C"][:, split:],
              z=c["z"][:, split:], h0=l1)
    y2, l2 = _run_ssd(ssd, c2)
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y) and np.array_equal(l2, last)


def check_ssd_free_decay(ssd, seed=94):
    """With no input the state only decays: S_L = exp(A sum dt) h0 and
    y_t = (C_t . (exp(A S_t) h0[p, :])) silu(z_t) in closed form."""
    c = _ssd_case(seed)
    c["x"] = np.zeros_like(c["x"])
    y, last = _run_ssd(ssd, c, softplus=True)
    dt = _softplus_np(c["dt"] + c["dt_bias"][None, None, :])             # (b, L, H)
    S = np.cumsum(dt, axis=1)
    decay = np.exp(c["A"][None, None, :] * S)                              # (b, L, H)
    hpg = c["x"].shape[2] // c["B"].shape[2]
    Cg = np.repeat(c["C"], hpg, axis=2)                                    # (b, L, H, N)
    want = decay[..., None] * np.einsum("blhn,bhpn->blhp", Cg, c["h0"]) * (c["z"] * expit(c["z"]))
    assert _rel(y, want) < 1e-12
    assert _rel(last, decay[:, -1][:, :, None, None] * c["h0"]) < 1e-13


SSD_CHECKS = [check_ssd_semiseparable, check_ssd_composition, check_ssd_free_decay]
SSD_SCAN_CHECKS = [check_ssd_is_broadcast_scan]


# --- gradients of the scan ------------------------------------------------------------------
# scan_from(u, x, A, B, C, D, z, bias, softplus, h0) -> (y, last_state)
# scan_bwd(u, x, A, B, C, dy, D, z, bias, softplus, h0, dlast) -> dict of gradients

def _bwd_case(seed, full):
    rng = _rng(seed)
    b, L, D, N = 2, 14, 3, 4
    c = dict(u=rng.standard_normal((b, L, D)), x=0.5 * rng.standard_normal((b, L, D)),
             A=-np.exp(rng.normal(0.0, 0.5, (D, N))), B=rng.standard_normal((b, L, N)),
             C=rng.standard_normal((b, L, N)), D=None, z=None, bias=None, h0=None, dlast=None,
             softplus=full)
    if full:
        c.update(D=rng.standard_normal(D), z=rng.standard_normal((b, L, D)), bias=rng.uniform(-1.0, 0.0, D),
                 h0=rng.standard_normal((b, D, N)), dlast=rng.standard_normal((b, D, N)))
    else:
        c["x"] = np.abs(c["x"]) + 0.05          # without softplus the step size itself stays positive
    c["dy"] = rng.standard_normal((b, L, D))
    return c, rng


def _check_bwd_fd(scan_from, scan_bwd, seed, full):
    """Every gradient against a central difference of the forward (fp64, eps = 1e-6) along a
    random direction: the loss is sum(dy * y) + sum(dlast * last_state)."""
    c, rng = _bwd_case(seed, full)
    g = scan_bwd(c["u"], c["x"], c["A"], c["B"], c["C"], c["dy"], c["D"], c["z"], c["bias"], c["softplus"],
                 c["h0"], c["dlast"])

    def loss(**kw):
        a = dict(c)
        a.update(kw)
        y, last = scan_from(a["u"], a["x"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["softplus"],
                            a["h0"])
        val = np.sum(c["dy"] * y)
        if c["dlast"] is not None:
            val += np.sum(c["dlast"] * last)
        return val

    pairs = [("u", "du"), ("x", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC")]
    if full:
        pairs += [("D", "dD"), ("z", "dz"), ("bias", "ddelta_bias"), ("h0", "dh0")]
    eps = 1e-6
    for name, gk in pairs:
        V = rng.standard_normal(np.shape(c[name]))
        fd = (loss(**{name: c[name] + eps * V}) - loss(**{name: c[name] - eps * V})) / (2 * eps)
        an = float(np.sum(g[gk] * V))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def check_bwd_fd_all_inputs(scan_from, scan_bwd):
    _check_bwd_fd(scan_from, scan_bwd, 71, True)


def check_bwd_fd_plain(scan_from, scan_bwd):
    _check_bwd_fd(scan_from, scan_bwd, 72, False)


def check_bwd_closed_forms(scan_from, scan_bwd):
    """dD = sum over batch and tokens of dy silu(z) u (the skip term is linear in D); with
    C = 0 and no dlast nothing flows back through the state: dB = dA = 0, ddelta = 0 and
    du = D dy silu(z)."""
    c, _ = _bwd_case(73, True)
    c["C"] = np.zeros_like(c["C"])
    g = scan_bwd(c["u"], c["x"], c["A"], c["B"], c["C"], c["dy"], c["D"], c["z"], c["bias"], True, c["h0"], None)
    gate = c["z"] / (1.0 + np.exp(-c["z"]))
    assert _rel(g["dD"], np.sum(c["dy"] * gate * c["u"], axis=(0, 1))) < 1e-13
    assert np.all(g["dB"] == 0.0) and np.all(g["dA"] == 0.0) and np.all(g["ddelta"] == 0.0)
    assert np.all(g["dh0"] == 0.0)
    assert _rel(g["du"], c["D"] * c["dy"] * gate) < 1e-13


BWD_CHECKS = [check_bwd_fd_all_inputs, check_bwd_fd_plain, check_bwd_closed_forms]


# --- gradients under the exact zero-order hold ------------------------------------------------
# scan_from_zoh / scan_bwd_zoh: as scan_from / scan_bwd with the input term
# (exp(delta A) - 1) / A * B * u (azimuth.plus/paper/mamba, Theorem 1's exact discretisation).

def check_bwd_zoh_fd_all_inputs(scan_from_zoh, scan_bwd_zoh):
    """Every gradient against central differences of the ZOH forward (A ~ -1: the closed form
    of d coefficient / dA)."""
    _check_bwd_fd(scan_from_zoh, scan_bwd_zoh, 74, True)


def check_bwd_zoh_fd_plain(scan_from_zoh, scan_bwd_zoh):
    _check_bwd_fd(scan_from_zoh, scan_bwd_zoh, 75, False)


def check_bwd_zoh_fd_small_A(scan_from_zoh, scan_bwd_zoh, seed=76):
    """Entries of A exactly 0, of size 1e-5 and of size 1e-3 (|delta A| from 1e-6 to a few
    1e-3: both sides of the series branch of d coefficient / dA), against central differences
    of the forward (whose coefficient is expm1 based there); the step along A is 1e-8."""
    c, rng = _bwd_case(seed, True)
    A = c["A"].copy()
    A[:, 0] = 0.0
    A[:, 1] = A[:, 1] * 1e-5
    A[:, 2:] = A[:, 2:] * 1e-3
    c["A"] = A
    g = scan_bwd_zoh(c["u"], c["x"], c["A"], c["B"], c["C"], c["dy"], c["D"], c["z"], c["bias"], True,
                     c["h0"], c["dlast"])

    def loss(A_):
        y, last = scan_from_zoh(c["u"], c["x"], A_, c["B"], c["C"], c["D"], c["z"], c["bias"], True, c["h0"])
        return np.sum(c["dy"] * y) + np.sum(c["dlast"] * last)
    eps = 1e-8
    for n in range(A.shape[1]):
        V = np.zeros_like(A)
        V[:, n] = rng.standard_normal(A.shape[0])
        fd = (loss(A + eps * V) - loss(A - eps * V)) / (2 * eps)
        an = float(np.sum(g["dA"] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (n, fd, an)


def check_bwd_zoh_zero_A(scan_from_zoh, scan_bwd_zoh, scan_bwd, seed=77):
    """At A = 0 the exact-ZOH coefficient is delta itself and the decay 1, so every gradient
    equals the simplified form's except dA, which gains d coefficient / dA = delta^2 / 2:
    dA_zoh - dA = sum over batch and tokens of lambda_t delta_t^2 / 2 B_t u_t, with lambda_t
    = the full gradient w.r.t. h_t (= sum_{s >= t} C_s dp_s + dlast, no decay at A = 0)."""
    c, _ = _bwd_case(seed, True)
    c["A"] = np.zeros_like(c["A"])
    args = (c["u"], c["x"], c["A"], c["B"], c["C"], c["dy"], c["D"], c["z"], c["bias"], True, c["h0"], c["dlast"])
    gz, gs = scan_bwd_zoh(*args), scan_bwd(*args)
    for k in gs:
        if k != "dA":
            assert _rel(gz[k], gs[k]) < 1e-12, k
    dt = _softplus_np(c["x"] + c["bias"])
    dp = c["dy"] * c["z"] / (1.0 + np.exp(-c["z"]))                       # (b, L, D)
    cdp = c["C"][:, :, None, :] * dp[:, :, :, None]                        # (b, L, D, N)
    lam = np.flip(np.cumsum(np.flip(cdp, axis=1), axis=1), axis=1) + c["dlast"][:, None, :, :]
    extra = np.sum(lam * (0.5 * dt * dt * c["u"])[:, :, :, None] * c["B"][:, :, None, :], axis=(0, 1))
    assert _rel(gz["dA"] - gs["dA"], extra) < 1e-10


BWD_ZOH_CHECKS = [check_bwd_zoh_fd_all_inputs, check_bwd_zoh_fd_plain, check_bwd_zoh_fd_small_A]



# --- sequences of different lengths -------------------------------------------------------------
# scan_varlen(u, x, A, B, C, lens, D, z, bias, softplus, h0) -> (y with NaN past each length,
# last_state); scan_from as above.

def _varlen_case(seed, bsz=4, L=37, D=3, N=4):
    rng = _rng(seed)
    c = dict(u=rng.standard_normal((bsz, L, D)), x=0.5 * rng.standard_normal((bsz, L, D)),
             A=-np.exp(rng.normal(0.0, 0.5, (D, N))), B=rng.standard_normal((bsz, L, N)),
             C=rng.standard_normal((bsz, L, N)), D=rng.standard_normal(D), z=rng.standard_normal((bsz, L, D)),
             bias=rng.uniform(-1.0, 0.0, D), h0=rng.standard_normal((bsz, D, N)))
    return c, rng


def _vl(scan_varlen, c, lens, **kw):
    a = dict(c)
    a.update(kw)
    return scan_varlen(a["u"], a["x"], a["A"], a["B"], a["C"], lens, a["D"], a["z"], a["bias"], True, a["h0"])


def check_varlen_full_lengths(scan_from, scan_varlen):
    """Every length = L: the batch scan itself, bitwise."""
    c, _ = _varlen_case(101)
    L = c["u"].shape[1]
    y, last = _vl(scan_varlen, c, [L] * c["u"].shape[0])
    y0, last0 = scan_from(c["u"], c["x"], c["A"], c["B"], c["C"], c["D"], c["z"], c["bias"], True, c["h0"])
    assert np.array_equal(y, y0) and np.array_equal(last, last0)


def check_varlen_padding_ignored(scan_from, scan_varlen):
    """Values past a sequence's length (here huge and NaN) change nothing: they are never read."""
    c, rng = _varlen_case(102)
    lens = [0, 1, 20, c["u"].shape[1]]
    y, last = _vl(scan_varlen, c, lens)
    d = {k: np.array(c[k], dtype=np.float64) for k in ("u", "x", "B", "C", "z")}
    for b, lb in enumerate(lens):
        for k in d:
            d[k][b, lb:] = np.nan if k in ("u", "B") else 1e30
    y2, last2 = _vl(scan_varlen, c, lens, **d)
    assert np.array_equal(y, y2, equal_nan=True) and np.array_equal(last, last2)
    for b, lb in enumerate(lens):
        assert np.all(np.isnan(y[b, lb:])) and np.all(np.isfinite(y[b, :lb]))


def check_varlen_continuation(scan_from, scan_varlen):
    """The state after a sequence's length, carried on over its remaining tokens, gives the
    full sequence's outputs and final state (within fp64 rounding), and its outputs up to the
    length are the full scan's: the lengths cut the recurrence, nothing else."""
    c, _ = _varlen_case(103)
    L = c["u"].shape[1]
    lens = [3, 17, 30, 36]
    y, last = _vl(scan_varlen, c, lens)
    y0, last0 = scan_from(c["u"], c["x"], c["A"], c["B"], c["C"], c["D"], c["z"], c["bias"], True, c["h0"])
    for b, lb in enumerate(lens):
        assert _rel(y[b, :lb], y0[b, :lb]) < 1e-14
        sl = (slice(b, b + 1), slice(lb, L))
        yr, lr = scan_from(c["u"][sl], c["x"][sl], c["A"], c["B"][sl], c["C"][sl], c["D"], c["z"][sl], c["bias"],
                           True, last[b:b + 1])
        assert _rel(yr[0], y0[b, lb:]) < 1e-12 and _rel(lr[0], last0[b]) < 1e-12


def check_varlen_zero_length(scan_from, scan_varlen):
    """Length 0: the final state is the initial one (zero without it), no output."""
    c, _ = _varlen_case(104)
    y, last = _vl(scan_varlen, c, [0, 0, 0, 0])
    assert np.array_equal(last, c["h0"]) and np.all(np.isnan(y))
    y, last = _vl(scan_varlen, c, [0, 5, 0, 2], h0=None)
    assert np.all(last[0] == 0.0) and np.all(last[2] == 0.0)


VARLEN_CHECKS = [check_varlen_full_lengths, check_varlen_padding_ignored, check_varlen_continuation,
                 check_varlen_zero_length]



# --- gradients of the variable-length scan ---------------------------------------------------------
# scan_bwd_varlen(u, x, A, B, C, dy, lens, D, z, bias, softplus, h0, dlast) -> dict of gradients

def _vl_bwd(scan_bwd_varlen, c, dy, lens, dlast, **kw):
    a = dict(c)
    a.update(kw)
    return scan_bwd_varlen(a["u"], a["x"], a["A"], a["B"], a["C"], dy, lens, a["D"], a["z"], a["bias"], True,
                           a["h0"], dlast)


def check_bwd_varlen_fd(scan_varlen, scan_bwd_varlen, seed=121):
    """Every gradient against central differences of the variable-length forward (a loss on
    y up to each length and on the state after it), lengths 0, 1, ragged and L."""
    c, rng = _varlen_case(seed, bsz=4, L=23, D=3, N=4)
    L = c["u"].shape[1]
    lens = np.array([0, 1, 14, L])
    dy = rng.standard_normal(c["u"].shape)
    dlast = rng.standard_normal(c["h0"].shape)
    g = _vl_bwd(scan_bwd_varlen, c, dy, lens, dlast)

    def loss(**kw):
        y, last = _vl(scan_varlen, c, lens, **kw)
        return np.nansum(dy * np.nan_to_num(y, nan=0.0)) + np.sum(dlast * last)
    eps = 1e-6
    for name, key in (("u", "du"), ("x", "ddelta"), ("z", "dz"), ("B", "dB"), ("C", "dC"), ("h0", "dh0"),
                      ("A", "dA"), ("D", "dD"), ("bias", "ddelta_bias")):
        V = rng.standard_normal(np.shape(c[name]))
        fd = (loss(**{name: c[name] + eps * V}) - loss(**{name: c[name] - eps * V})) / (2 * eps)
        an = float(np.sum(g[key] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def check_bwd_varlen_full_lengths(scan_bwd, scan_bwd_varlen, seed=122):
    """All lengths L: the batch backward exactly (same arithmetic per sequence)."""
    c, rng = _varlen_case(seed)
    L = c["u"].shape[1]
    dy = rng.standard_normal(c["u"].shape)
    dlast = rng.standard_normal(c["h0"].shape)
    g = _vl_bwd(scan_bwd_varlen, c, dy, [L] * c["u"].shape[0], dlast)
    g0 = scan_bwd(c["u"], c["x"], c["A"], c["B"], c["C"], dy, c["D"], c["z"], c["bias"], True, c["h0"], dlast)
    for k in g0:
        assert _rel(g[k], g0[k]) < 1e-13, k


def check_bwd_varlen_padding(scan_bwd, scan_bwd_varlen, seed=123):
    """Values past each length, in the inputs and in dy, change no gradient; the gradients
    there are exactly zero."""
    c, rng = _varlen_case(seed)
    lens = [0, 1, 20, c["u"].shape[1]]
    dy = rng.standard_normal(c["u"].shape)
    dlast = rng.standard_normal(c["h0"].shape)
    g = _vl_bwd(scan_bwd_varlen, c, dy, lens, dlast)
    d = {k: np.array(c[k], dtype=np.float64) for k in ("u", "x", "B", "C", "z")}
    dy2 = dy.copy()
    for b, lb in enumerate(lens):
        for k in d:
            d[k][b, lb:] = 1e30 if k in ("x", "z") else -7.5
        dy2[b, lb:] = 1e30
    g2 = _vl_bwd(scan_bwd_varlen, c, dy2, lens, dlast, **d)
    for k in g:
        assert np.array_equal(g[k], g2[k]), k
    for b, lb in enumerate(lens):
        for k in ("du", "ddelta", "dz", "dB", "dC"):
            assert np.all(g[k][b, lb:] == 0.0), (k, b)
    assert np.array_equal(g["dh0"][0], dlast[0])   # length 0: the adjoint passes straight through


BWD_VARLEN_CHECKS = [check_bwd_varlen_full_lengths, check_bwd_varlen_padding]
