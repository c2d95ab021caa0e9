"""Each plausible mistake planted in a copy of the oracle (on the CPU) must be caught by
at least one of the pins in pins.py: a dropped term, a wrong sign, a wrong index, a
transposed operand.  The copies are compiled into a temporary directory; the real oracle
is never modified."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ssm_oracle.c")

MUTANTS = {
    "drop_skip_term": ("if (Dv) yt = yt + Dv[d] * ut;", "if (Dv) yt = yt;"),
    "wrong_sign_of_A": ("double dA = exp(dt * A[d * N + n]);\n                    h[n]",
                        "double dA = exp(-dt * A[d * N + n]);\n                    h[n]"),
    "reversed_state_index_of_A": ("double dA = exp(dt * A[d * N + n]);\n                    h[n]",
                                  "double dA = exp(dt * A[d * N + (N - 1 - n)]);\n                    h[n]"),
    "swap_B_and_C": ("const double *Bt = B + (b * L + t) * N;\n            const double *Ct = C + (b * L + t) * N;",
                     "const double *Bt = C + (b * L + t) * N;\n            const double *Ct = B + (b * L + t) * N;"),
    "drop_delta_bias": ("if (delta_bias) x = x + delta_bias[d];", "if (delta_bias) x = x;"),
    "no_softplus": ("double dt = softplus_flag ? oracle_softplus(x) : x;", "double dt = x;"),
    "drop_gate": ("if (z) yt = yt * oracle_silu(z[i]);", "if (z) yt = yt;"),
    "sigmoid_not_silu": ("return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    "previous_token_input": ("h[n] = dA * h[n] + dt * Bt[n] * ut;",
                             "h[n] = dA * h[n] + dt * Bt[n] * u[t > 0 ? i - D : i];"),
    "drop_delta_in_input_term": ("h[n] = dA * h[n] + dt * Bt[n] * ut;", "h[n] = dA * h[n] + Bt[n] * ut;"),
    "readout_before_update": ("h[n] = dA * h[n] + dt * Bt[n] * ut;\n                }\n            }\n            double acc = 0.0;\n            for (int64_t n = 0; n < N; ++n) acc = acc + Ct[n] * h[n];",
                              "(void)dA;\n                }\n            }\n            double acc = 0.0;\n            for (int64_t n = 0; n < N; ++n) acc = acc + Ct[n] * h[n];\n            if (!zoh) for (int64_t n = 0; n < N; ++n) h[n] = exp(dt * A[d * N + n]) * h[n] + dt * Bt[n] * ut;"),
    "last_state_wrong_index": ("last_state[(b * D + d) * N + n] = h[n];", "last_state[(b * D + d) * N + n] = h[0];"),
    "softplus_wrong_branch": ("if (x > 0.0) return x + log1p(exp(-x));", "if (x > 0.0) return x + log1p(exp(x));"),
    "ignore_initial_state": ("h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;", "h[n] = 0.0;"),
    "bwd_adjoint_without_decay": ("G[n] = a * lam;", "G[n] = lam;"),
    "bwd_drop_input_term_of_ddelta": ("dd = dd + lam * (A[d * N + n] * a * hprev + dm_ddt * Bt[n] * ut);",
                                      "dd = dd + lam * (A[d * N + n] * a * hprev);"),
    "bwd_zoh_coefficient_derivative_one": ("double dm_ddt = zoh ? a : 1.0;", "double dm_ddt = 1.0;"),
    "bwd_zoh_no_coefficient_term_in_dA": (
        "if (zoh) dA[d * N + n] += lam * oracle_zoh_coef_da(dt[t], A[d * N + n]) * Bt[n] * ut;", ""),
    "bwd_zoh_dB_with_delta": ("dBl[(b * L + t) * N + n] += lam * m * ut;", "dBl[(b * L + t) * N + n] += lam * dt[t] * ut;"),
    "bwd_zoh_du_with_delta": ("du_t = du_t + lam * m * Bt[n];", "du_t = du_t + lam * dt[t] * Bt[n];"),
    "bwd_zoh_coefficient_derivative_sign": ("return (dt * exp(x) - expm1(x) / a) / a;",
                                            "return (expm1(x) / a - dt * exp(x)) / a;"),
    "bwd_zoh_series_second_term": ("return dt * dt * (0.5 + x * (1.0 / 3.0 + x * (1.0 / 8.0 + x * (1.0 / 30.0 + x / 144.0))));",
                                   "return dt * dt * (0.5 + x * (1.0 / 2.0 + x * (1.0 / 8.0 + x * (1.0 / 30.0 + x / 144.0))));"),
    "bwd_zoh_series_limit": ("return dt * dt * (0.5 + x * (1.0 / 3.0 + x * (1.0 / 8.0 + x * (1.0 / 30.0 + x / 144.0))));",
                             "return dt * (0.5 + x * (1.0 / 3.0 + x * (1.0 / 8.0 + x * (1.0 / 30.0 + x / 144.0))));"),
    "bwd_current_state_for_previous": ("double hprev = t > 0 ? hist[(t - 1) * N + n] : hinit[n];",
                                       "double hprev = hist[t * N + n];"),
    "bwd_no_softplus_derivative": ("double dx = softplus_flag ? dd * oracle_sigmoid(x) : dd;", "double dx = dd;"),
    "bwd_dC_from_adjoint": ("dCl[(b * L + t) * N + n] += dp * hist[t * N + n];",
                            "dCl[(b * L + t) * N + n] += lam * hist[t * N + n];"),
    "bwd_gate_derivative_missing_term": ("dz[i] = dy[i] * p * (sg * (1.0 + z[i] * (1.0 - sg)));",
                                         "dz[i] = dy[i] * p * sg;"),
    "zoh_simplified_coefficient": ("return a != 0.0 ? expm1(dt * a) / a : dt;", "return dt;"),
    "zoh_exp_for_expm1": ("return a != 0.0 ? expm1(dt * a) / a : dt;", "return a != 0.0 ? exp(dt * a) / a : dt;"),
    "zoh_wrong_limit": ("return a != 0.0 ? expm1(dt * a) / a : dt;", "return a != 0.0 ? expm1(dt * a) / a : 0.0;"),
    "zoh_decay_from_coefficient": ("h[n] = exp(dt * a) * h[n] + oracle_zoh_coef(dt, a) * Bt[n] * ut;",
                                   "h[n] = exp(-dt * a) * h[n] + oracle_zoh_coef(dt, a) * Bt[n] * ut;"),
    "conv_reversed_taps": ("acc = acc + w[d * width + k] * hist[t + k];",
                           "acc = acc + w[d * width + (width - 1 - k)] * hist[t + k];"),
    "conv_window_one_late": ("acc = acc + w[d * width + k] * hist[t + k];",
                             "acc = acc + w[d * width + k] * hist[t + k > 0 ? t + k - 1 : 0];"),
    "conv_drop_bias": ("double acc = bias ? bias[d] : 0.0;", "double acc = 0.0;"),
    "conv_drop_silu": ("out[(b * L + t) * D + d] = silu ? oracle_silu(acc) : acc;",
                       "out[(b * L + t) * D + d] = acc;"),
    "conv_ignore_state": ("hist[r] = state ? state[(b * H + r) * D + d] : 0.0;", "hist[r] = 0.0;"),
    "conv_bwd_no_silu_derivative": ("g[t] = go * (s * (1.0 + pre * (1.0 - s)));", "g[t] = go * s;"),
    "conv_bwd_reversed_taps_dx": ("dhist[t + k] = dhist[t + k] + w[d * width + k] * g[t];",
                                  "dhist[t + k] = dhist[t + k] + w[d * width + (width - 1 - k)] * g[t];"),
    "conv_bwd_dw_input_one_late": ("dw[d * width + k] = dw[d * width + k] + g[t] * hist[t + k];",
                                   "dw[d * width + k] = dw[d * width + k] + g[t] * hist[t + k > 0 ? t + k - 1 : 0];"),
    "conv_bwd_dstate_newest_rows": ("dstate[(b * H + r) * D + d] = dhist[r];",
                                    "dstate[(b * H + r) * D + d] = dhist[r + 1];"),
    "conv_bwd_dbias_from_dout": ("if (dbias) dbias[d] = dbias[d] + g[t];",
                                 "if (dbias) dbias[d] = dbias[d] + dout[(b * L + t) * D + d];"),
    "conv_state_out_oldest_rows": ("state_out[(b * H + r) * D + d] = hist[L + r];",
                                   "state_out[(b * H + r) * D + d] = hist[r];"),
    "ssd_group_index": ("g = h / hpg;", "g = h % G;"),
    "ssd_drop_dt_in_input": ("s[n] = dA * s[n] + dt * x[i] * Bt[n];", "s[n] = dA * s[n] + x[i] * Bt[n];"),
    "ssd_decay_without_dt": ("double dA = exp(dt * A[h]);", "double dA = exp(A[h]);"),
    "ssd_readout_with_B": ("acc = acc + Ct[n] * s[n];", "acc = acc + Bt[n] * s[n];"),
    "decay_squared": ("h[n] = dA * h[n] + dt * Bt[n] * ut;", "h[n] = dA * dA * h[n] + dt * Bt[n] * ut;"),
}


def _build_mutant(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation {name} does not apply"
    text = text.replace(old, new, 1)
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    so = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O1", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11", str(src),
                    "-o", str(so), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    lib.ssm_oracle_scan.argtypes = [I64, I64, I64, I64, P, P, P, P, P, P, P, P, ctypes.c_int, P, P, ctypes.c_int]
    lib.ssm_oracle_scan.restype = ctypes.c_int
    lib.ssm_oracle_scan_from.argtypes = [I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, ctypes.c_int, P, P,
                                         ctypes.c_int]
    lib.ssm_oracle_scan_from.restype = ctypes.c_int
    lib.ssm_oracle_scan_bwd.argtypes = [I64, I64, I64, I64] + [P] * 9 + [ctypes.c_int] + [P] * 11 + [ctypes.c_int]
    lib.ssm_oracle_scan_bwd.restype = ctypes.c_int
    lib.ssm_oracle_conv1d.argtypes = [I64, I64, I64, I64, P, P, P, P, ctypes.c_int, P, P]
    lib.ssm_oracle_conv1d.restype = ctypes.c_int
    lib.ssm_oracle_conv1d_bwd.argtypes = [I64, I64, I64, I64, P, P, P, P, ctypes.c_int, P, P, P, P, P]
    lib.ssm_oracle_conv1d_bwd.restype = ctypes.c_int
    lib.ssm_oracle_ssd.argtypes = [I64] * 6 + [P] * 9 + [ctypes.c_int, P, P, ctypes.c_int]
    lib.ssm_oracle_ssd.restype = ctypes.c_int

    def f64(a):
        return None if a is None else np.ascontiguousarray(a, dtype=np.float64)

    def ptr(a):
        return None if a is None else a.ctypes.data

    def scan(u, x, A, B, C, D, z, bias, softplus):
        u, x, A, B, C, D, z, bias = map(f64, (u, x, A, B, C, D, z, bias))
        bsz, L, Dch = u.shape
        N = A.shape[1]
        y = np.empty((bsz, L, Dch))
        h = np.empty((bsz, Dch, N))
        lib.ssm_oracle_scan(bsz, L, Dch, N, ptr(u), ptr(x), ptr(A), ptr(B), ptr(C), ptr(D), ptr(z),
                            ptr(bias), int(bool(softplus)), ptr(y), ptr(h), 1)
        return y, h

    def scan_from(u, x, A, B, C, D, z, bias, softplus, h0):
        u, x, A, B, C, D, z, bias, h0 = map(f64, (u, x, A, B, C, D, z, bias, h0))
        bsz, L, Dch = u.shape
        N = A.shape[1]
        y = np.empty((bsz, L, Dch))
        h = np.empty((bsz, Dch, N))
        lib.ssm_oracle_scan_from(bsz, L, Dch, N, ptr(h0), ptr(u), ptr(x), ptr(A), ptr(B), ptr(C), ptr(D),
                                 ptr(z), ptr(bias), int(bool(softplus)), ptr(y), ptr(h), 1)
        return y, h
    def scan_from_zoh(u, x, A, B, C, D, z, bias, softplus, h0):
        u, x, A, B, C, D, z, bias, h0 = map(f64, (u, x, A, B, C, D, z, bias, h0))
        bsz, L, Dch = u.shape
        N = A.shape[1]
        y = np.empty((bsz, L, Dch))
        h = np.empty((bsz, Dch, N))
        lib.ssm_oracle_scan_from(bsz, L, Dch, N, ptr(h0), ptr(u), ptr(x), ptr(A), ptr(B), ptr(C), ptr(D),
                                 ptr(z), ptr(bias), int(bool(softplus)) | 2, ptr(y), ptr(h), 1)
        return y, h

    def scan_zoh(u, x, A, B, C, D, z, bias, softplus):
        u, x, A, B, C, D, z, bias = map(f64, (u, x, A, B, C, D, z, bias))
        bsz, L, Dch = u.shape
        N = A.shape[1]
        y = np.empty((bsz, L, Dch))
        h = np.empty((bsz, Dch, N))
        lib.ssm_oracle_scan(bsz, L, Dch, N, ptr(u), ptr(x), ptr(A), ptr(B), ptr(C), ptr(D), ptr(z),
                            ptr(bias), int(bool(softplus)) | 2, ptr(y), ptr(h), 1)
        return y, h

    def scan_bwd(u, x, A, B, C, dy, D, z, bias, softplus, h0, dlast, zoh=False):
        u, x, A, B, C, dy, D, z, bias, h0, dlast = map(f64, (u, x, A, B, C, dy, D, z, bias, h0, dlast))
        bsz, L, Dch = u.shape
        N = A.shape[1]
        out = dict(du=np.empty((bsz, L, Dch)), ddelta=np.empty((bsz, L, Dch)), dA=np.empty((Dch, N)),
                   dB=np.empty((bsz, L, N)), dC=np.empty((bsz, L, N)), dD=np.empty(Dch),
                   dz=np.empty((bsz, L, Dch)), ddelta_bias=np.empty(Dch), dh0=np.empty((bsz, Dch, N)))
        lib.ssm_oracle_scan_bwd(bsz, L, Dch, N, ptr(h0), ptr(u), ptr(x), ptr(A), ptr(B), ptr(C), ptr(D), ptr(z),
                                ptr(bias), int(bool(softplus)) | (2 if zoh else 0), ptr(dy), ptr(dlast),
                                ptr(out["du"]),
                                ptr(out["ddelta"]), ptr(out["dA"]), ptr(out["dB"]), ptr(out["dC"]), ptr(out["dD"]),
                                ptr(out["dz"]), ptr(out["ddelta_bias"]), ptr(out["dh0"]), 1)
        return out
    def conv(x, w, bias, state, silu):
        x, w, bias, state = map(f64, (x, w, bias, state))
        bsz, L, Dch = x.shape
        width = w.shape[1]
        out = np.empty((bsz, L, Dch))
        st = np.empty((bsz, width - 1, Dch))
        lib.ssm_oracle_conv1d(bsz, L, Dch, width, ptr(x), ptr(w), ptr(bias), ptr(state), int(bool(silu)), ptr(out),
                              ptr(st))
        return out, st
    def conv_bwd(x, w, dout, bias, state, silu):
        x, w, dout, bias, state = map(f64, (x, w, dout, bias, state))
        bsz, L, Dch = x.shape
        width = w.shape[1]
        out = dict(dx=np.empty((bsz, L, Dch)), dw=np.empty((Dch, width)), dbias=np.empty(Dch),
                   dstate=np.empty((bsz, width - 1, Dch)))
        lib.ssm_oracle_conv1d_bwd(bsz, L, Dch, width, ptr(x), ptr(w), ptr(bias), ptr(state), int(bool(silu)),
                                  ptr(dout), ptr(out["dx"]), ptr(out["dw"]), ptr(out["dbias"]), ptr(out["dstate"]))
        return out
    def ssd(x, dt, A, B, C, D, z, dt_bias, softplus, h0):
        x, dt, A, B, C, D, z, dt_bias, h0 = map(f64, (x, dt, A, B, C, D, z, dt_bias, h0))
        bsz, L, H, Pd = x.shape
        G, N = B.shape[2], B.shape[3]
        y = np.empty((bsz, L, H, Pd))
        last = np.empty((bsz, H, Pd, N))
        lib.ssm_oracle_ssd(bsz, L, H, Pd, G, N, ptr(h0), ptr(x), ptr(dt), ptr(A), ptr(B), ptr(C), ptr(D), ptr(z),
                           ptr(dt_bias), int(bool(softplus)), ptr(y), ptr(last), 1)
        return y, last
    def scan_bwd_zoh(*a):
        return scan_bwd(*a, zoh=True)
    return scan, scan_from, scan_bwd, scan_zoh, conv, conv_bwd, ssd, scan_from_zoh, scan_bwd_zoh


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    (scan, scan_from, scan_bwd, scan_zoh, conv, conv_bwd, ssd, scan_from_zoh,
     scan_bwd_zoh) = _build_mutant(tmp_path, name, old, new)
    caught = []
    with np.errstate(all="ignore"):
        for check in pins.ALL_CHECKS:
            try:
                check(scan)
            except AssertionError:
                caught.append(check.__name__)
        for check in pins.H0_CHECKS:
            try:
                check(scan_from)
            except AssertionError:
                caught.append(check.__name__)
        for check in pins.ZOH_CHECKS:
            try:
                check(scan_zoh)
            except AssertionError:
                caught.append(check.__name__)
        for check in pins.CONV_CHECKS:
            try:
                check(conv)
            except AssertionError:
                caught.append(check.__name__)
        for check in pins.CONV_BWD_CHECKS:
            try:
                check(conv, conv_bwd)
            except AssertionError:
                caught.append(check.__name__)
        for check in pins.SSD_CHECKS:
            try:
                check(ssd)
            except AssertionError:
                caught.append(check.__name__)
        for check in pins.SSD_SCAN_CHECKS:
            try:
                check(ssd, scan_from)
            except AssertionError:
                caught.append(check.__name__)
        for check in pins.BWD_CHECKS:
            try:
                check(scan_from, scan_bwd)
            except AssertionError:
                caught.append(check.__name__)
        for check in pins.BWD_ZOH_CHECKS:
            try:
                check(scan_from_zoh, scan_bwd_zoh)
            except AssertionError:
                caught.append(check.__name__)
        try:
            pins.check_bwd_zoh_zero_A(scan_from_zoh, scan_bwd_zoh, scan_bwd)
        except AssertionError:
            caught.append("check_bwd_zoh_zero_A")
    assert caught, f"mutant {name} passed every pin"
