"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import numpy as np
import pytest

import pins


def _scan(oracle_mod):
    def f(u, x, A, B, C, D, z, bias, softplus):
        return oracle_mod.scan(u, x, A, B, C, D=D, z=z, delta_bias=bias, softplus=softplus, threads=2)
    return f


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(oracle_mod, check):
    check(_scan(oracle_mod))


def _scan_zoh(oracle_mod):
    def f(u, x, A, B, C, D, z, bias, softplus):
        return oracle_mod.scan(u, x, A, B, C, D=D, z=z, delta_bias=bias, softplus=softplus, threads=2,
                               exact_zoh=True)
    return f


@pytest.mark.parametrize("check", pins.ZOH_CHECKS, ids=lambda c: c.__name__)
def test_oracle_zoh_pin(oracle_mod, check):
    check(_scan_zoh(oracle_mod))


def _conv(oracle_mod):
    def f(x, w, bias, state, silu):
        return oracle_mod.conv1d(x, w, bias=bias, state=state, silu=silu)
    return f


@pytest.mark.parametrize("check", pins.CONV_CHECKS, ids=lambda c: c.__name__)
def test_oracle_conv_pin(oracle_mod, check):
    check(_conv(oracle_mod))


def _conv_bwd(oracle_mod):
    def f(x, w, dout, bias, state, silu):
        return oracle_mod.conv1d_bwd(x, w, dout, bias=bias, state=state, silu=silu)
    return f


@pytest.mark.parametrize("check", pins.CONV_BWD_CHECKS, ids=lambda c: c.__name__)
def test_oracle_conv_bwd_pin(oracle_mod, check):
    check(_conv(oracle_mod), _conv_bwd(oracle_mod))


def _ssd(oracle_mod):
    def f(x, dt, A, B, C, D, z, dt_bias, softplus, h0):
        return oracle_mod.ssd(x, dt, A, B, C, D=D, z=z, dt_bias=dt_bias, softplus=softplus, h0=h0, threads=2)
    return f


def _scan_from(oracle_mod):
    def f(u, x, A, B, C, D, z, bias, softplus, h0):
        return oracle_mod.scan(u, x, A, B, C, D=D, z=z, delta_bias=bias, softplus=softplus, threads=2, h0=h0)
    return f


@pytest.mark.parametrize("check", pins.SSD_CHECKS, ids=lambda c: c.__name__)
def test_oracle_ssd_pin(oracle_mod, check):
    check(_ssd(oracle_mod))


@pytest.mark.parametrize("check", pins.SSD_SCAN_CHECKS, ids=lambda c: c.__name__)
def test_oracle_ssd_scan_pin(oracle_mod, check):
    check(_ssd(oracle_mod), _scan_from(oracle_mod))



def test_step_repeated_equals_scan(oracle_mod):
    """Recurrent form == scan form (urworte.de "Methodische Grundlagen"; shakilmahmud.com
    section 3): L single-token steps from a zero state reproduce the scan bitwise when the
    step size is already activated (softplus off, no bias)."""
    rng = np.random.default_rng(31)
    S, L, D, N = 3, 40, 6, 5
    u = rng.standard_normal((S, L, D))
    dt = np.logaddexp(0.0, rng.standard_normal((S, L, D)))
    A = -np.exp(rng.normal(1.0, 0.5, (D, N)))
    B = rng.standard_normal((S, L, N))
    C = rng.standard_normal((S, L, N))
    Dv = rng.standard_normal(D)
    z = rng.standard_normal((S, L, D))
    y_scan, h_scan = oracle_mod.scan(u, dt, A, B, C, D=Dv, z=z, delta_bias=None, softplus=False)
    st = np.zeros((S, D, N))
    for t in range(L):
        y_t, st = oracle_mod.step(st, u[:, t], dt[:, t], A, B[:, t], C[:, t], D=Dv, z=z[:, t])
        assert np.array_equal(y_t, y_scan[:, t])
    assert np.array_equal(st, h_scan)


def test_step_from_nonzero_state_closed_form(oracle_mod):
    """One step from a given state: h' = exp(delta A) h + delta B u, y = (C.h' + D u) silu(z),
    evaluated here with numpy broadcasting."""
    rng = np.random.default_rng(32)
    S, D, N = 4, 7, 16
    st = 0.1 * rng.standard_normal((S, D, N))
    u = rng.standard_normal((S, D))
    dt = np.logaddexp(0.0, rng.standard_normal((S, D)) - 2)
    A = -np.exp(rng.normal(np.log(4), 0.5, (D, N)))
    B = rng.standard_normal((S, N))
    C = rng.standard_normal((S, N))
    Dv = rng.standard_normal(D)
    z = rng.standard_normal((S, D))
    y, st2 = oracle_mod.step(st, u, dt, A, B, C, D=Dv, z=z)
    h = np.exp(dt[:, :, None] * A[None]) * st + (dt * u)[:, :, None] * B[:, None, :]
    want = (np.einsum("sdn,sn->sd", h, C) + Dv[None] * u) * z / (1 + np.exp(-z))
    np.testing.assert_allclose(st2, h, rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-15)


def test_oracle_thread_count_invariant(oracle_mod):
    """Channels are independent: the result does not depend on how they are spread over
    threads (bitwise)."""
    from selective_state_space_32_amd import inputs
    c = inputs.scan_case(2, 64, 37, 16, "bf16", gate=True, seed=3)
    y1, h1 = oracle_mod.scan_case(c, threads=1)
    y2, h2 = oracle_mod.scan_case(c, threads=4)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


def test_oracle_channel_sampling_exact(oracle_mod):
    """Sampling channels evaluates exactly the full-problem values of those channels."""
    from selective_state_space_32_amd import inputs
    c = inputs.scan_case(2, 50, 33, 8, "f32", gate=True, seed=4)
    y, h = oracle_mod.scan_case(c)
    sel = np.array([0, 5, 17, 32])
    ys, hs = oracle_mod.scan_case(c, channels=sel)
    assert np.array_equal(ys, y[:, :, sel]) and np.array_equal(hs, h[:, sel])


def test_oracle_rejects_bad_n(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.scan(np.ones((1, 2, 1)), np.ones((1, 2, 1)), np.ones((1, 300)),
                        np.ones((1, 2, 300)), np.ones((1, 2, 300)))


def _scan_from(oracle_mod):
    def f(u, x, A, B, C, D, z, bias, softplus, h0):
        return oracle_mod.scan(u, x, A, B, C, D=D, z=z, delta_bias=bias, softplus=softplus, h0=h0)
    return f


@pytest.mark.parametrize("check", pins.H0_CHECKS, ids=lambda c: c.__name__)
def test_h0_pins(oracle_mod, check):
    check(_scan_from(oracle_mod))


def test_scan_from_state_equals_steps(oracle_mod):
    """The recurrent form (shakilmahmud.com section 3): L oracle steps from a state equal the
    oracle scan from that state (step sizes already activated, no bias)."""
    rng = np.random.default_rng(54)
    S, L, Dch, N = 2, 12, 3, 4
    u = rng.standard_normal((S, L, Dch))
    dt = np.log1p(np.exp(0.5 * rng.standard_normal((S, L, Dch))))
    A = -np.exp(rng.normal(0.3, 0.5, (Dch, N)))
    B = rng.standard_normal((S, L, N))
    C = rng.standard_normal((S, L, N))
    Dv = rng.standard_normal(Dch)
    z = rng.standard_normal((S, L, Dch))
    h0 = rng.standard_normal((S, Dch, N))
    y, last = oracle_mod.scan(u, dt, A, B, C, D=Dv, z=z, softplus=False, h0=h0)
    st = h0.copy()
    for t in range(L):
        yt, st = oracle_mod.step(st, u[:, t], dt[:, t], A, B[:, t], C[:, t], D=Dv, z=z[:, t])
        assert np.array_equal(yt, y[:, t])
    assert np.array_equal(st, last)


def _scan_bwd(oracle_mod):
    def f(u, x, A, B, C, dy, D, z, bias, softplus, h0, dlast):
        return oracle_mod.scan_bwd(u, x, A, B, C, dy, D=D, z=z, delta_bias=bias, softplus=softplus, h0=h0,
                                   dlast=dlast)
    return f


@pytest.mark.parametrize("check", pins.BWD_CHECKS, ids=lambda c: c.__name__)
def test_bwd_pins(oracle_mod, check):
    check(_scan_from(oracle_mod), _scan_bwd(oracle_mod))


def _scan_from_zoh(oracle_mod):
    def f(u, x, A, B, C, D, z, bias, softplus, h0):
        return oracle_mod.scan(u, x, A, B, C, D=D, z=z, delta_bias=bias, softplus=softplus, threads=2, h0=h0,
                               exact_zoh=True)
    return f


def _scan_bwd_zoh(oracle_mod):
    def f(u, x, A, B, C, dy, D, z, bias, softplus, h0, dlast):
        return oracle_mod.scan_bwd(u, x, A, B, C, dy, D=D, z=z, delta_bias=bias, softplus=softplus, h0=h0,
                                   dlast=dlast, exact_zoh=True)
    return f


@pytest.mark.parametrize("check", pins.BWD_ZOH_CHECKS, ids=lambda c: c.__name__)
def test_bwd_zoh_pins(oracle_mod, check):
    check(_scan_from_zoh(oracle_mod), _scan_bwd_zoh(oracle_mod))


def test_bwd_zoh_zero_A(oracle_mod):
    pins.check_bwd_zoh_zero_A(_scan_from_zoh(oracle_mod), _scan_bwd_zoh(oracle_mod), _scan_bwd(oracle_mod))


def _scan_varlen(oracle_mod):
    def f(u, x, A, B, C, lens, D, z, bias, softplus, h0):
        return oracle_mod.scan_varlen(u, x, A, B, C, lens, D=D, z=z, delta_bias=bias, softplus=softplus, threads=2,
                                      h0=h0)
    return f


@pytest.mark.parametrize("check", pins.VARLEN_CHECKS, ids=lambda c: c.__name__)
def test_varlen_pins(oracle_mod, check):
    check(_scan_from(oracle_mod), _scan_varlen(oracle_mod))


def _scan_bwd_varlen(oracle_mod):
    def f(u, x, A, B, C, dy, lens, D, z, bias, softplus, h0, dlast):
        return oracle_mod.scan_bwd_varlen(u, x, A, B, C, dy, lens, D=D, z=z, delta_bias=bias, softplus=softplus,
                                          h0=h0, dlast=dlast, threads=2)
    return f


def test_bwd_varlen_fd(oracle_mod):
    pins.check_bwd_varlen_fd(_scan_varlen(oracle_mod), _scan_bwd_varlen(oracle_mod))


@pytest.mark.parametrize("check", pins.BWD_VARLEN_CHECKS, ids=lambda c: c.__name__)
def test_bwd_varlen_pins(oracle_mod, check):
    check(_scan_bwd(oracle_mod), _scan_bwd_varlen(oracle_mod))
