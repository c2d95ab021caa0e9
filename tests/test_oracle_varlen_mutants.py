"""Plausible mistakes in the variable-length scan and its gradients (the per-sequence loops of
oracle.scan_varlen and oracle.scan_bwd_varlen), each planted in a copy written here on top of
the oracle's pinned scan and backward: every one must fail at least one of the pins in
pins.py.  The real oracle is never modified."""
import numpy as np
import pytest

import pins


def _fwd_mutant(oracle_mod, kind):
    def scan_varlen(u, x, A, B, C, lens, D, z, bias, softplus, h0):
        u = np.asarray(u, np.float64)
        bsz, L, Dch = u.shape
        N = np.asarray(A).shape[1]
        y = np.full((bsz, L, Dch), np.nan)
        last = np.empty((bsz, Dch, N))
        for b in range(bsz):
            lb = int(min(max(int(lens[b]), 0), L))
            if kind == "length_plus_one":
                lb = min(lb + 1, L)
            if kind == "length_minus_one":
                lb = max(lb - 1, 0)
            hb_src = b if kind != "initial_state_of_next_sequence" else (b + 1) % bsz
            hb = None if h0 is None else np.asarray(h0, np.float64)[hb_src:hb_src + 1]
            if lb == 0:
                last[b] = 0.0 if (hb is None or kind == "zero_length_drops_state") else hb[0]
                continue
            n_in = L if kind == "reads_past_the_length" else lb
            sl = (slice(b, b + 1), slice(0, n_in))
            yb, lsb = oracle_mod.scan(u[sl], np.asarray(x)[sl], A, np.asarray(B)[sl], np.asarray(C)[sl], D=D,
                                      z=None if z is None else np.asarray(z)[sl], delta_bias=bias, softplus=softplus,
                                      h0=hb, threads=2)
            y[b, :lb] = yb[0, :lb]
            if kind == "final_state_of_the_whole_row":
                _, lsb = oracle_mod.scan(u[b:b + 1], np.asarray(x)[b:b + 1], A, np.asarray(B)[b:b + 1],
                                         np.asarray(C)[b:b + 1], D=D,
                                         z=None if z is None else np.asarray(z)[b:b + 1], delta_bias=bias,
                                         softplus=softplus, h0=hb, threads=2)
            last[b] = lsb[0]
        return y, last
    return scan_varlen


def _bwd_mutant(oracle_mod, kind):
    def scan_bwd_varlen(u, x, A, B, C, dy, lens, D, z, bias, softplus, h0, dlast):
        u = np.asarray(u, np.float64)
        bsz, L, Dch = u.shape
        N = np.asarray(A).shape[1]
        out = dict(du=np.zeros((bsz, L, Dch)), ddelta=np.zeros((bsz, L, Dch)), dA=np.zeros((Dch, N)),
                   dB=np.zeros((bsz, L, N)), dC=np.zeros((bsz, L, N)), dh0=np.zeros((bsz, Dch, N)))
        if D is not None:
            out["dD"] = np.zeros(Dch)
        if z is not None:
            out["dz"] = np.zeros((bsz, L, Dch))
        if bias is not None:
            out["ddelta_bias"] = np.zeros(Dch)
        for b in range(bsz):
            lb = int(min(max(int(lens[b]), 0), L))
            if kind == "length_minus_one":
                lb = max(lb - 1, 0)
            dl_b = None if (dlast is None or kind == "dlast_ignored") else np.asarray(dlast, np.float64)[b:b + 1]
            if lb == 0:
                if dl_b is not None and kind != "zero_length_drops_adjoint":
                    out["dh0"][b] = dl_b[0]
                continue
            n_in = L if kind == "gradients_of_the_whole_row" else lb
            sl = (slice(b, b + 1), slice(0, n_in))
            h0_b = np.zeros((1, Dch, N)) if h0 is None else np.asarray(h0, np.float64)[b:b + 1]
            dyb = np.asarray(dy)[sl]
            g = oracle_mod.scan_bwd(u[sl], np.asarray(x)[sl], A, np.asarray(B)[sl], np.asarray(C)[sl], dyb, D=D,
                                    z=None if z is None else np.asarray(z)[sl], delta_bias=bias, softplus=softplus,
                                    h0=h0_b, dlast=dl_b, threads=2)
            for k in ("du", "ddelta", "dB", "dC") + (("dz",) if z is not None else ()):
                out[k][b, :n_in] = g[k][0]
            for k in ("dA",) + (("dD",) if D is not None else ()) + (("ddelta_bias",) if bias is not None else ()):
                if kind == "sums_of_the_first_sequence_only" and b > 0:
                    continue
                out[k] += g[k]
            out["dh0"][b] = g["dh0"][0]
        return out
    return scan_bwd_varlen


def _scan_from(oracle_mod):
    def f(u, x, A, B, C, D, z, bias, softplus, h0):
        return oracle_mod.scan(u, x, A, B, C, D=D, z=z, delta_bias=bias, softplus=softplus, h0=h0, threads=2)
    return f


def _scan_bwd(oracle_mod):
    def f(u, x, A, B, C, dy, D, z, bias, softplus, h0, dlast):
        return oracle_mod.scan_bwd(u, x, A, B, C, dy, D=D, z=z, delta_bias=bias, softplus=softplus, h0=h0,
                                   dlast=dlast, threads=2)
    return f


def _scan_varlen(oracle_mod):
    def f(u, x, A, B, C, lens, D, z, bias, softplus, h0):
        return oracle_mod.scan_varlen(u, x, A, B, C, lens, D=D, z=z, delta_bias=bias, softplus=softplus, h0=h0,
                                      threads=2)
    return f


FWD_MUTANTS = ["length_plus_one", "length_minus_one", "initial_state_of_next_sequence", "zero_length_drops_state",
               "final_state_of_the_whole_row", "reads_past_the_length"]
BWD_MUTANTS = ["length_minus_one", "dlast_ignored", "zero_length_drops_adjoint", "gradients_of_the_whole_row",
               "sums_of_the_first_sequence_only"]


def _caught(checks):
    caught = []
    for name, run in checks:
        try:
            run()
        except (AssertionError, ValueError, IndexError):
            caught.append(name)
    return caught


@pytest.mark.parametrize("kind", FWD_MUTANTS)
def test_varlen_forward_mistake_is_caught(oracle_mod, kind):
    mutant = _fwd_mutant(oracle_mod, kind)
    checks = [(c.__name__, lambda c=c: c(_scan_from(oracle_mod), mutant)) for c in pins.VARLEN_CHECKS]
    assert _caught(checks), f"no pin catches the planted mistake {kind}"


@pytest.mark.parametrize("kind", BWD_MUTANTS)
def test_varlen_backward_mistake_is_caught(oracle_mod, kind):
    mutant = _bwd_mutant(oracle_mod, kind)
    checks = [(c.__name__, lambda c=c: c(_scan_bwd(oracle_mod), mutant)) for c in pins.BWD_VARLEN_CHECKS]
    checks.append(("check_bwd_varlen_fd", lambda: pins.check_bwd_varlen_fd(_scan_varlen(oracle_mod), mutant)))
    assert _caught(checks), f"no pin catches the planted mistake {kind}"


def test_unmutated_copies_pass(oracle_mod):
    """The copies above without a planted mistake pass every pin (so a catch is the mistake's)."""
    for c in pins.VARLEN_CHECKS:
        c(_scan_from(oracle_mod), _fwd_mutant(oracle_mod, "none"))
    for c in pins.BWD_VARLEN_CHECKS:
        c(_scan_bwd(oracle_mod), _bwd_mutant(oracle_mod, "none"))
    pins.check_bwd_varlen_fd(_scan_varlen(oracle_mod), _bwd_mutant(oracle_mod, "none"))
