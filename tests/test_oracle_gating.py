"""Pins of the oracle's gate computation (g = -exp(A_log) softplus(a + dt_bias),
beta = sigmoid(b), page "[Qwen3.5][Feature] support fla triton kernel for
qwen3.5", "Usage or Command" item 5), CPU only.

Each pin is a function of a gating implementation, so the same pins are shown
to reject planted mistakes (mutants written here) as well as to accept the
oracle.
"""
import math

import numpy as np
import pytest

import oracle


def pin_worked_points(gate):
    # A_log = 0, dt_bias = 0, a = 0: g = -ln 2; b = 0: beta = 1/2
    g, beta = gate(np.zeros(1), np.zeros(1), np.zeros((1, 1)), np.zeros((1, 1)))
    assert abs(g[0, 0] + math.log(2.0)) < 1e-15 and abs(beta[0, 0] - 0.5) < 1e-15
    # A_log = ln 3, dt_bias = 1/2, a = ln(e^2 - 1) - 1/2: softplus = 2, g = -6
    a = math.log(math.e ** 2 - 1.0) - 0.5
    g, _ = gate(np.array([math.log(3.0)]), np.array([0.5]), np.array([[a]]), np.zeros((1, 1)))
    assert abs(g[0, 0] + 6.0) < 1e-13
    # beta(ln 3) = 3/4, beta(-ln 3) = 1/4
    _, beta = gate(np.zeros(1), np.zeros(1), np.zeros((2, 1)), np.array([[math.log(3.0)], [-math.log(3.0)]]))
    assert abs(beta[0, 0] - 0.75) < 1e-15 and abs(beta[1, 0] - 0.25) < 1e-15


def pin_per_head_axis(gate):
    # three value heads with different A_log / dt_bias: column j uses entry j
    A_log = np.array([0.0, math.log(2.0), math.log(5.0)])
    dt = np.array([0.0, 1.0, -2.0])
    a = np.array([[0.0, -1.0, 2.0], [1.0, 0.0, 0.0]])
    g, _ = gate(A_log, dt, a, np.zeros_like(a))
    for t in range(2):
        for j in range(3):
            x = a[t, j] + dt[j]
            assert abs(g[t, j] + math.exp(A_log[j]) * math.log1p(math.exp(x))) < 1e-14


def pin_identities(gate):
    x = np.concatenate([np.linspace(-40, 40, 801), [-700.0, -100.0, 100.0, 700.0]])
    z = np.zeros(1)
    g_p, s_p = gate(z, z, x[:, None], x[:, None])
    g_m, s_m = gate(z, z, -x[:, None], -x[:, None])
    sp_p, sp_m = -g_p[:, 0], -g_m[:, 0]            # A_log = 0: g = -softplus
    assert np.all(np.isfinite(sp_p)) and np.all(sp_p > 0) and np.all(np.isfinite(s_p))
    assert np.max(np.abs((sp_p - sp_m) - x) / np.maximum(1.0, np.abs(x))) < 1e-14   # sp(x) - sp(-x) = x
    assert np.max(np.abs(s_p + s_m - 1.0)) < 1e-15                                  # s(x) + s(-x) = 1
    # d softplus / dx = sigmoid (central differences away from the tails)
    h = 1e-5
    xs = np.linspace(-8, 8, 33)
    gp, s = gate(z, z, (xs + h)[:, None], xs[:, None])
    gm, _ = gate(z, z, (xs - h)[:, None], xs[:, None])
    assert np.max(np.abs((gm - gp)[:, 0] / (2 * h) - s[:, 0])) < 1e-9
    # tails: softplus(50) = 50 + e^-50, softplus(-50) = e^-50
    gt, _ = gate(z, z, np.array([[50.0], [-50.0]]), np.zeros((2, 1)))
    assert abs(-gt[0, 0] - 50.0) < 1e-13 and abs(-gt[1, 0] / math.exp(-50.0) - 1.0) < 1e-12


def pin_library(gate):
    # moderate arguments: the textbook formulas through Python's math module
    rng = np.random.default_rng(0)
    A_log = rng.uniform(0, math.log(16), 4)
    dt = rng.uniform(0, 1, 4)
    a = rng.normal(size=(5, 4))
    b = rng.normal(0, 2, size=(5, 4))
    g, beta = gate(A_log, dt, a, b)
    for t in range(5):
        for j in range(4):
            ge = -math.exp(A_log[j]) * math.log(1.0 + math.exp(a[t, j] + dt[j]))
            be = 1.0 / (1.0 + math.exp(-b[t, j]))
            assert abs(g[t, j] - ge) <= 1e-14 * abs(ge) and abs(beta[t, j] - be) <= 1e-15


PINS = [pin_worked_points, pin_per_head_axis, pin_identities, pin_library]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_gating_pins(pin):
    pin(oracle.gating)


def _mutant(kind):
    def gate(A_log, dt_bias, a, b):
        A_log, dt_bias, a, b = (np.asarray(x, dtype=np.float64) for x in (A_log, dt_bias, a, b))
        x = a if kind == "no_dt_bias" else a + dt_bias
        sp = np.exp(x) if kind == "exp_for_softplus" else oracle.softplus(x)
        A = A_log if kind == "A_log_not_exponentiated" else np.exp(A_log)
        if kind == "head_axis_reversed":
            A = A[::-1]
        g = A * sp if kind == "positive_g" else -A * sp
        beta = oracle.sigmoid(-b if kind == "sigmoid_of_minus_b" else b)
        if kind == "beta_is_b":
            beta = b
        return g, beta
    return gate


MUTANTS = ["no_dt_bias", "exp_for_softplus", "A_log_not_exponentiated", "head_axis_reversed",
           "positive_g", "sigmoid_of_minus_b", "beta_is_b"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_gating_pins_reject_mutants(kind):
    gate = _mutant(kind)
    failed = 0
    for pin in PINS:
        try:
            pin(gate)
        except AssertionError:
            failed += 1
    assert failed >= 1, f"mutant {kind} passed every pin"


def test_recurrent_gated_is_recurrent_of_the_gates():
    rng = np.random.default_rng(1)
    B, T, H, HV, K, V = 1, 9, 1, 2, 4, 3
    q = rng.normal(size=(B, T, H, K)).astype(np.float32)
    k = rng.normal(size=(B, T, H, K)).astype(np.float32)
    v = rng.normal(size=(B, T, HV, V)).astype(np.float32)
    a = rng.normal(size=(B, T, HV)).astype(np.float32)
    b = rng.normal(size=(B, T, HV)).astype(np.float32)
    A_log = np.array([0.3, 1.7], np.float32)
    dt = np.array([0.2, 0.9], np.float32)
    o1, f1 = oracle.recurrent_gated(q, k, v, A_log, dt, a, b, use_l2norm=True)
    g, beta = oracle.gating(A_log, dt, a, b)
    o2, f2 = oracle.recurrent(q, k, v, g.astype(np.float32), beta.astype(np.float32), use_l2norm=True)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)
    # b -> -inf: beta = 0, the state only decays (no write)
    s0 = rng.normal(size=(1, HV, K, V)).astype(np.float32)
    _, f3 = oracle.recurrent_gated(q, k, v, A_log, dt, a, np.full_like(b, -800.0), initial_state=s0)
    gsum = oracle.gating(A_log, dt, a, b)[0].astype(np.float32).astype(np.float64).sum(axis=1)[0]
    assert np.allclose(f3[0], s0[0] * np.exp(gsum)[:, None, None], rtol=1e-12, atol=0)
