"""The discriminating bf16 parity cases reject every planted mistake.

For each mutant of ``test_oracle_mutants`` (a plain numpy loop of the
recurrence with one deliberate error), run on exactly the inputs of the
discriminating GPU parity cases (``parity_cases``): the mutant's distance from
the correct recurrence must be at least five times the case's bar in at least
one case, so that the bf16 kernel test would fail on a kernel with that
mistake.  The correct loop itself agrees with the C oracle to 1e-12.
"""
import numpy as np
import pytest
import torch

import oracle
from parity_cases import BASE
from test_oracle_mutants import MUTANTS, py_recurrent
from workloads import make_inputs

MARGIN = 5.0


def _inputs(w):
    x = oracle.add_gates(make_inputs(w, seed=0, io_dtype=torch.float32))
    f = lambda t: t[0].numpy().astype(np.float64)   # first sequence, every head
    return x, f(x["q"]), f(x["k"]), f(x["v"]), f(x["g"]), f(x["beta"]), x["initial_state"][0].numpy()


_CACHE = {}


def _control(name):
    if name not in _CACHE:
        w = BASE[name][0]
        x, q, k, v, g, beta, s0 = _inputs(w)
        o, fin = py_recurrent(q, k, v, g, beta, x["scale"], w.use_l2norm, s0)
        _CACHE[name] = (x, q, k, v, g, beta, s0, o, fin)
    return _CACHE[name]


@pytest.mark.parametrize("name", list(BASE))
def test_control_matches_oracle(name):
    x, q, k, v, g, beta, s0, o, fin = _control(name)
    o_ref, f_ref = oracle.recurrent(x["q"][:1], x["k"][:1], x["v"][:1], x["g"][:1], x["beta"][:1],
                                    scale=x["scale"], use_l2norm=x["use_l2norm"],
                                    initial_state=x["initial_state"][:1])
    np.testing.assert_allclose(o, o_ref[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(fin, f_ref[0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("norm", [True, False], ids=["l2norm", "no_l2norm"])
@pytest.mark.parametrize("mutant", MUTANTS)
def test_mutant_misses_bf16_bars(mutant, norm):
    """Each family of cases (with and without the L2 norm, which the kernel
    runs through different code) rejects every mutant on its own."""
    powers = {}
    for name, (w, bar_o, bar_s) in BASE.items():
        if w.use_l2norm != norm:
            continue
        x, q, k, v, g, beta, s0, o, fin = _control(name)
        om, fm = py_recurrent(q, k, v, g, beta, x["scale"], norm, s0, mutant)
        d_o, d_s = float(np.abs(om - o).max()), float(np.abs(fm - fin).max())
        powers[name] = max(d_o / bar_o, d_s / bar_s)
        print(f"{mutant} on {name}: max|do| {d_o:.3g} (bar {bar_o}), max|dS| {d_s:.3g} (bar {bar_s})")
    assert powers and max(powers.values()) >= MARGIN, f"{mutant}: largest miss {max(powers.values()):.2f}x the bar"
