"""Pins of the oracle's gate-input gradients (oracle.gating_bwd), CPU only.

The gates are g = -exp(A_log) softplus(a + dt_bias) and beta = sigmoid(b) (page
"[Qwen3.5][Feature] support fla triton kernel for qwen3.5", "Usage or Command"
item 5); the gradients of a, b, A_log and dt_bias follow from them by the chain
rule.  The pins hold any implementation to central finite differences of the
forward gate function, to hand-worked points and to the sum structure over the
head axis; planted mistakes are shown to fail them.
"""
import math

import numpy as np
import pytest

import oracle


def _loss_grads_fd(A_log, dt, a, b, dg, dbeta, h=1e-6):
    """Central differences of L = sum(dg * g) + sum(dbeta * beta) with respect to
    every input, through the forward gate function only."""
    def L(A_log, dt, a, b):
        g, beta = oracle.gating(A_log, dt, a, b)
        return float(np.sum(dg * g) + np.sum(dbeta * beta))

    out = []
    for idx, x in enumerate((a, b, A_log, dt)):
        gx = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            k = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[k] += h
            xm[k] -= h
            args_p = [a, b, A_log, dt]
            args_m = [a, b, A_log, dt]
            args_p[idx], args_m[idx] = xp, xm
            gx[k] = (L(args_p[2], args_p[3], args_p[0], args_p[1]) - L(args_m[2], args_m[3], args_m[0], args_m[1])) / (2 * h)
        out.append(gx)
    return out   # da, db, dA_log, ddt_bias


def pin_finite_differences(gate_bwd):
    rng = np.random.default_rng(0)
    A_log = rng.uniform(0, math.log(16), 3)
    dt = rng.uniform(0, 1, 3)
    a = rng.normal(size=(4, 3))
    b = rng.normal(0, 2, size=(4, 3))
    dg = rng.normal(size=(4, 3))
    dbeta = rng.normal(size=(4, 3))
    got = gate_bwd(A_log, dt, a, b, dg, dbeta)
    want = _loss_grads_fd(A_log, dt, a, b, dg, dbeta)
    for name, x, y in zip(("da", "db", "dA_log", "ddt_bias"), got, want):
        assert np.max(np.abs(x - y)) <= 1e-7 * max(1.0, np.max(np.abs(y))), name


def pin_worked_points(gate_bwd):
    # A_log = 0, dt_bias = 0, a = 0: g = -ln 2, dg/da = -sigmoid(0) = -1/2;
    # b = 0: beta = 1/2, dbeta/db = 1/4; A_log = ln 3, a = dt = 0: dg/da = -3/2
    one = np.ones((1, 1))
    da, db, dA, ddt = gate_bwd(np.zeros(1), np.zeros(1), np.zeros((1, 1)), np.zeros((1, 1)), 2 * one, 4 * one)
    assert abs(da[0, 0] + 1.0) < 1e-15 and abs(db[0, 0] - 1.0) < 1e-15
    assert abs(dA[0] + 2 * math.log(2.0)) < 1e-15 and abs(ddt[0] + 1.0) < 1e-15
    da, _, dA, _ = gate_bwd(np.array([math.log(3.0)]), np.zeros(1), np.zeros((1, 1)), np.zeros((1, 1)), one, one)
    assert abs(da[0, 0] + 1.5) < 1e-15 and abs(dA[0] + 3 * math.log(2.0)) < 1e-14
    # b = ln 3: beta = 3/4, beta (1 - beta) = 3/16
    _, db, _, _ = gate_bwd(np.zeros(1), np.zeros(1), np.zeros((1, 1)), np.array([[math.log(3.0)]]), one, one)
    assert abs(db[0, 0] - 3.0 / 16.0) < 1e-15


def pin_head_sums(gate_bwd):
    # dA_log and ddt_bias sum over every row, separately per head; a leading
    # batch axis is just more rows
    rng = np.random.default_rng(1)
    A_log, dt = rng.normal(size=2), rng.normal(size=2)
    a, b, dg, dbeta = (rng.normal(size=(2, 3, 2)) for _ in range(4))
    da, db, dA, ddt = gate_bwd(A_log, dt, a, b, dg, dbeta)
    g, _ = oracle.gating(A_log, dt, a, b)
    for j in range(2):
        assert abs(ddt[j] - da[..., j].sum()) < 1e-13
        assert abs(dA[j] - (dg[..., j] * g[..., j]).sum()) < 1e-13
    # one row at a time gives the same per-row gradients
    da1, db1, _, _ = gate_bwd(A_log, dt, a[1, 2:3], b[1, 2:3], dg[1, 2:3], dbeta[1, 2:3])
    assert np.array_equal(da1[0], da[1, 2]) and np.array_equal(db1[0], db[1, 2])


PINS = [pin_finite_differences, pin_worked_points, pin_head_sums]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_gating_bwd_pins(pin):
    pin(oracle.gating_bwd)


def _mutant(kind):
    def gate_bwd(A_log, dt, a, b, dg, dbeta):
        A_log, dt, a, b, dg, dbeta = (np.asarray(x, dtype=np.float64) for x in (A_log, dt, a, b, dg, dbeta))
        g, beta = oracle.gating(A_log, dt, a, b)
        x = a if kind == "no_dt_bias_in_derivative" else a + dt
        d = oracle.softplus(x) if kind == "softplus_for_sigmoid" else oracle.sigmoid(x)
        da = dg * (np.exp(A_log) * d if kind == "sign" else -np.exp(A_log) * d)
        db = dbeta * (beta if kind == "beta_for_derivative" else beta * (1.0 - beta))
        HV = A_log.shape[0]
        dA = (dg * (g if kind != "dA_without_g" else 1.0)).reshape(-1, HV).sum(axis=0)
        ddt = da.reshape(-1, HV).sum(axis=0)
        if kind == "ddt_last_row_only":
            ddt = da.reshape(-1, HV)[-1]
        return da, db, dA, ddt
    return gate_bwd


MUTANTS = ["no_dt_bias_in_derivative", "softplus_for_sigmoid", "sign", "beta_for_derivative", "dA_without_g",
           "ddt_last_row_only"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_gating_bwd_pins_reject_mutants(kind):
    fn = _mutant(kind)
    failed = 0
    for pin in PINS:
        try:
            pin(fn)
        except AssertionError:
            failed += 1
    assert failed >= 1, f"mutant {kind} passed every pin"
