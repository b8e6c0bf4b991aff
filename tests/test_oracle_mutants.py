"""Planted mistakes: each mutant of the recurrence (a plain numpy loop written
here, on the CPU) must be rejected by the pins and by the float32 parity gate.

The control (no mutation) must agree with the C oracle to rounding, so the
mutants differ from the oracle only by their planted mistake.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, make_inputs, scaled

MUTANTS = ["no_delta", "drop_initial_state", "undecayed_erase", "gate_shifted",
           "read_before_write", "interleaved_gva", "beta_one", "scale_one", "transposed_read"]


def py_recurrent(q, k, v, g, beta, scale, use_l2norm, S0, mutant=None):
    """q, k [T,H,K]; v [T,HV,V]; g, beta [T,HV]; S0 [HV,K,V] or None."""
    T, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    G = HV // H
    o = np.zeros((T, HV, V))
    fin = np.zeros((HV, K, V))
    for j in range(HV):
        jk = (j % H) if mutant == "interleaved_gva" else j // G
        S = np.zeros((K, V)) if (S0 is None or mutant == "drop_initial_state") else S0[j].astype(np.float64).copy()
        for t in range(T):
            qh, kh = q[t, jk].astype(np.float64), k[t, jk].astype(np.float64)
            if use_l2norm:
                qh = qh / np.sqrt(qh @ qh + 1e-6)
                kh = kh / np.sqrt(kh @ kh + 1e-6)
            tg = t - 1 if mutant == "gate_shifted" else t
            a = np.exp(g[tg, j]) if tg >= 0 else 1.0
            b = 1.0 if mutant == "beta_one" else float(beta[t, j])
            sc = 1.0 if mutant == "scale_one" else scale
            if mutant == "read_before_write":
                o[t, j] = sc * (a * S).T @ qh
            Sprev = S
            S = a * S
            if mutant == "no_delta":
                d = b * v[t, j]
            elif mutant == "undecayed_erase":
                d = b * (v[t, j] - Sprev.T @ kh)
            else:
                d = b * (v[t, j] - S.T @ kh)
            S = S + np.outer(kh, d)
            if mutant == "transposed_read":
                o[t, j] = sc * S @ qh
            elif mutant != "read_before_write":
                o[t, j] = sc * S.T @ qh
        fin[j] = S
    return o, fin


def _case():
    # tiny-workload distributions, GVA and an initial state so every mutant has
    # something to break; 128 tokens keep the numpy loop fast
    w = scaled(WORKLOADS["gva"], "mut", B=1, T=128, H=2, HV=4, K=32, V=32)
    x = oracle.add_gates(make_inputs(w, seed=0, io_dtype=torch.float32))
    f = lambda t: t[0].numpy().astype(np.float64)
    return x, f(x["q"]), f(x["k"]), f(x["v"]), f(x["g"]), f(x["beta"]), x["initial_state"][0].numpy()


def test_control_matches_oracle():
    x, q, k, v, g, beta, s0 = _case()
    o_ref, f_ref = oracle.recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"], scale=x["scale"],
                                    use_l2norm=True, initial_state=x["initial_state"])
    o, fin = py_recurrent(q, k, v, g, beta, x["scale"], True, s0)
    np.testing.assert_allclose(o, o_ref[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(fin, f_ref[0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("mutant", MUTANTS)
def test_mutant_fails_fp32_gate(mutant):
    """The float32-mode gate (max-abs 1e-4 on o and on the final state)
    rejects every mutant on workload-like inputs."""
    x, q, k, v, g, beta, s0 = _case()
    o_ref, f_ref = oracle.recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"], scale=x["scale"],
                                    use_l2norm=True, initial_state=x["initial_state"])
    o, fin = py_recurrent(q, k, v, g, beta, x["scale"], True, s0, mutant)
    err = max(np.abs(o - o_ref[0]).max(), np.abs(fin - f_ref[0]).max())
    assert err > 1e-4, f"{mutant}: max error {err:.3g} would pass the 1e-4 gate"


@pytest.mark.parametrize("mutant", MUTANTS)
def test_mutant_fails_a_pin(mutant):
    """At least one of the hand-derived / closed-form pins rejects each mutant
    (run against the mutant instead of the oracle)."""
    failures = []
    # hand-worked examples
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "handworked.json")))["cases"]
    for c in cases:
        T, K, V = len(c["q"]), c["K"], c["V"]
        s0 = None if c["initial_state"] is None else np.array(c["initial_state"], float)[None]
        o, fin = py_recurrent(np.array(c["q"], float).reshape(T, 1, K), np.array(c["k"], float).reshape(T, 1, K),
                              np.array(c["v"], float).reshape(T, 1, V), np.array(c["g"], float).reshape(T, 1),
                              np.array(c["beta"], float).reshape(T, 1), c["scale"], c["use_l2norm"], s0, mutant)
        if (np.abs(o[:, 0] - np.array(c["o"])).max() > c["tol"]
                or np.abs(fin[0] - np.array(c["final_state"])).max() > c["tol"]):
            failures.append(c["name"])
    # grouped heads: v-head j must read key head j // G (contiguous groups)
    rng = np.random.default_rng(0)
    T, H, HV, K, V = 6, 2, 4, 3, 3
    q = rng.normal(size=(T, H, K)); k = rng.normal(size=(T, H, K)); v = rng.normal(size=(T, HV, V))
    g = -rng.uniform(0, 0.5, (T, HV)); beta = rng.uniform(0, 1, (T, HV))
    o, _ = py_recurrent(q, k, v, g, beta, 1.0, True, None, mutant)
    o2, _ = py_recurrent(np.repeat(q, 2, axis=1), np.repeat(k, 2, axis=1), v, g, beta, 1.0, True, None, None)
    if np.abs(o - o2).max() > 1e-12:
        failures.append("gva_repeat")
    # beta = 0 is pure decay of the initial state
    S0 = rng.normal(size=(HV, K, V))
    o, _ = py_recurrent(q, k, v, g, np.zeros_like(beta), 0.5, False, S0, mutant)
    G_ = np.cumsum(g, axis=0)
    for j in range(HV):
        want = 0.5 * np.exp(G_[:, j])[:, None] * (q[:, j // 2] @ S0[j])
        if np.abs(o[:, j] - want).max() > 1e-12:
            failures.append("beta_zero")
            break
    assert failures, f"{mutant} passed every pin"
