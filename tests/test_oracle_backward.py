"""Pins of the fp64 backward oracle (oracle/backward.py).

The backward is the hand-written chain rule of the token recurrence; it is
pinned to (1) central finite differences of the float64 forward recurrence,
which share none of its derivative algebra, over every input (q, k, v, g,
beta, initial state) with the L2 norm on and off, grouped value heads and
packed sequences; (2) the closed form of the no-write case (beta = 0), where
the state only decays; and the float64 forward itself is pinned to the C
oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.backward import backward, forward64


def _inputs(rng, B, T, H, HV, K, V, N=None):
    N = B if N is None else N
    return dict(q=rng.normal(0, 1, (B, T, H, K)), k=rng.normal(0, 1, (B, T, H, K)),
                v=rng.normal(0, 1, (B, T, HV, V)), g=-rng.uniform(0.05, 0.6, (B, T, HV)),
                beta=rng.uniform(0.1, 0.9, (B, T, HV)), h0=rng.normal(0, 0.5, (N, HV, K, V)),
                do=rng.normal(0, 1, (B, T, HV, V)), dht=rng.normal(0, 1, (N, HV, K, V)))


def _loss(x, scale, l2, cu):
    o, fin = forward64(x["q"], x["k"], x["v"], x["g"], x["beta"], scale=scale, use_l2norm=l2,
                       initial_state=x["h0"], cu_seqlens=cu)
    return float(np.sum(o * x["do"]) + np.sum(fin * x["dht"]))


CASES = {
    "gva_l2": dict(B=1, T=5, H=1, HV=2, K=3, V=2, l2=True, cu=None),
    "plain_batch": dict(B=2, T=4, H=2, HV=2, K=2, V=3, l2=False, cu=None),
    "varlen_l2": dict(B=1, T=6, H=1, HV=2, K=3, V=2, l2=True, cu=[0, 2, 2, 6]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_finite_differences(name):
    c = CASES[name]
    rng = np.random.default_rng(11)
    N = c["B"] if c["cu"] is None else len(c["cu"]) - 1
    x = _inputs(rng, c["B"], c["T"], c["H"], c["HV"], c["K"], c["V"], N=N)
    scale = 0.7
    cu = None if c["cu"] is None else np.array(c["cu"])
    grads = backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], dht=x["dht"], scale=scale,
                     use_l2norm=c["l2"], initial_state=x["h0"], cu_seqlens=cu)
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "h0": "dh0"}
    eps = 1e-6
    for inp, gname in names.items():
        a = x[inp]
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            old = a[idx]
            a[idx] = old + eps
            lp = _loss(x, scale, c["l2"], cu)
            a[idx] = old - eps
            lm = _loss(x, scale, c["l2"], cu)
            a[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grads[gname], fd, rtol=1e-6, atol=1e-7, err_msg=f"{name}: {gname}")


def test_no_write_closed_form():
    """beta = 0: S_t = exp(gamma_t) S0 with gamma_t the cumulative gate, so
    o_t = scale exp(gamma_t) S0^T q_t, nothing depends on k or v, and
    dS0 = sum_t scale exp(gamma_t) q_t do_t^T + exp(gamma_T) dS_T."""
    rng = np.random.default_rng(5)
    x = _inputs(rng, 1, 7, 1, 1, 4, 3)
    x["beta"][:] = 0.0
    s = 0.3
    gr = backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], dht=x["dht"], scale=s,
                  initial_state=x["h0"])
    gam = np.cumsum(x["g"][0, :, 0])
    S0, q, do = x["h0"][0, 0], x["q"][0, :, 0], x["do"][0, :, 0]
    dh0 = sum(s * np.exp(gam[t]) * np.outer(q[t], do[t]) for t in range(7)) + np.exp(gam[-1]) * x["dht"][0, 0]
    dq = np.stack([s * np.exp(gam[t]) * S0 @ do[t] for t in range(7)])
    np.testing.assert_allclose(gr["dh0"][0, 0], dh0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gr["dq"][0, :, 0], dq, rtol=1e-12, atol=1e-12)
    assert np.abs(gr["dk"]).max() == 0 and np.abs(gr["dv"]).max() == 0


def test_forward64_matches_c_oracle():
    rng = np.random.default_rng(3)
    x = _inputs(rng, 2, 9, 2, 4, 5, 3)
    f32 = {n: torch.tensor(x[n], dtype=torch.float32) for n in ("q", "k", "v", "g", "beta", "h0")}
    o_c, fin_c = oracle.recurrent(f32["q"], f32["k"], f32["v"], f32["g"], f32["beta"], scale=0.4,
                                  use_l2norm=True, initial_state=f32["h0"])
    o_p, fin_p = forward64(*(f32[n] for n in ("q", "k", "v", "g", "beta")), scale=0.4, use_l2norm=True,
                           initial_state=f32["h0"])
    np.testing.assert_allclose(o_p, o_c, rtol=0, atol=1e-12)
    np.testing.assert_allclose(fin_p, fin_c, rtol=0, atol=1e-12)
