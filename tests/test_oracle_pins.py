"""Pins of the fp64 oracle to facts fixed outside of it.

Each test checks the oracle (token recurrence in oracle/gdn_oracle.c) against
something other than itself: a hand-derived worked example, a closed form of a
special case, an invariant of the mathematics, the transition-matrix product
form of the recurrence, or the chunked (WY) form.  A plausible slip in the
oracle (dropped decay, transposed state, wrong head grouping, output read
before the write, missing delta term, wrong norm) fails at least one of them;
``test_oracle_mutants.py`` shows that.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.chunked import chunked_unit

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked.json")


def _t(a, shape=None):
    x = torch.tensor(np.asarray(a, dtype=np.float64), dtype=torch.float32)
    return x if shape is None else x.reshape(shape)


def _rand_inputs(rng, B, T, H, HV, K, V, qk_std=1.0, gmax=1.0):
    q = rng.normal(0, qk_std, (B, T, H, K)).astype(np.float32)
    k = rng.normal(0, qk_std, (B, T, H, K)).astype(np.float32)
    v = rng.normal(0, 1, (B, T, HV, V)).astype(np.float32)
    g = (-rng.uniform(0, gmax, (B, T, HV))).astype(np.float32)
    beta = rng.uniform(0, 1, (B, T, HV)).astype(np.float32)
    return q, k, v, g, beta


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_handworked_examples(case):
    K, V = case["K"], case["V"]
    T = len(case["q"])
    s0 = None if case["initial_state"] is None else _t(case["initial_state"], (1, 1, K, V))
    o, fin = oracle.recurrent(_t(case["q"], (1, T, 1, K)), _t(case["k"], (1, T, 1, K)),
                              _t(case["v"], (1, T, 1, V)), _t(case["g"], (1, T, 1)),
                              _t(case["beta"], (1, T, 1)), scale=case["scale"],
                              use_l2norm=case["use_l2norm"], initial_state=s0)
    tol = case["tol"]
    np.testing.assert_allclose(o[0, :, 0, :], np.array(case["o"]), rtol=0, atol=tol)
    np.testing.assert_allclose(fin[0, 0], np.array(case["final_state"]), rtol=0, atol=tol)


def test_transition_product_form():
    """S_T = P_{T..1} S0 + sum_t P_{T..t+1} beta_t k_t v_t^T with
    P_{b..a} = M_b ... M_a and M_t = exp(g_t) (I - beta_t k_t k_t^T), built
    from explicit K x K matrices; K != V so a transposed state cannot pass."""
    rng = np.random.default_rng(1)
    T, K, V = 9, 3, 5
    q, k, v, g, beta = _rand_inputs(rng, 1, T, 1, 1, K, V)
    S0 = rng.normal(0, 1, (1, 1, K, V)).astype(np.float32)
    scale = 0.7
    o, fin = oracle.recurrent(q, k, v, g, beta, scale=scale, initial_state=S0)
    kk, qq, vv = (x[0, :, 0].astype(np.float64) for x in (k, q, v))
    gg, bb = g[0, :, 0].astype(np.float64), beta[0, :, 0].astype(np.float64)
    M = [math.exp(gg[t]) * (np.eye(K) - bb[t] * np.outer(kk[t], kk[t])) for t in range(T)]
    for tt in range(1, T + 1):
        P = np.eye(K)
        for t in range(tt):
            P = M[t] @ P
        S = P @ S0[0, 0].astype(np.float64)
        for t in range(tt):
            Pt = np.eye(K)
            for s in range(t + 1, tt):
                Pt = M[s] @ Pt
            S = S + Pt @ np.outer(bb[t] * kk[t], vv[t])
        np.testing.assert_allclose(o[0, tt - 1, 0], scale * S.T @ qq[tt - 1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fin[0, 0], S, rtol=1e-12, atol=1e-12)


def test_beta_zero_is_pure_decay():
    """beta = 0: nothing is written, S_t = exp(G_t) S0 with G_t the gate
    cumsum from the sequence start, so o_t = scale exp(G_t) S0^T qh_t."""
    rng = np.random.default_rng(2)
    T, K, V = 37, 8, 6
    q, k, v, g, beta = _rand_inputs(rng, 1, T, 1, 1, K, V, gmax=0.3)
    beta[:] = 0
    S0 = rng.normal(0, 1, (1, 1, K, V)).astype(np.float32)
    o, fin = oracle.recurrent(q, k, v, g, beta, scale=0.5, use_l2norm=True, initial_state=S0)
    G = np.cumsum(g[0, :, 0].astype(np.float64))
    qq = q[0, :, 0].astype(np.float64)
    qh = qq / np.sqrt((qq * qq).sum(1, keepdims=True) + 1e-6)
    s0 = S0[0, 0].astype(np.float64)
    want = 0.5 * np.exp(G)[:, None] * (qh @ s0)
    np.testing.assert_allclose(o[0, :, 0], want, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fin[0, 0], math.exp(G[-1]) * s0, rtol=1e-12, atol=1e-14)
    # and with g = 0 as well: o_t = scale S0^T qh_t for every t
    g[:] = 0
    o, fin = oracle.recurrent(q, k, v, g, beta, scale=0.5, use_l2norm=True, initial_state=S0)
    np.testing.assert_allclose(o[0, :, 0], 0.5 * qh @ s0, rtol=1e-12, atol=1e-14)


def test_orthogonal_keys_give_linear_attention():
    """Distinct one-hot keys never overlap, so the erase term vanishes and
    the rule reduces to decayed linear attention:
    o_t = scale sum_{j<=t} exp(G_t - G_j) beta_j (q_t . k_j) v_j."""
    rng = np.random.default_rng(3)
    T, K, V = 12, 16, 7
    perm = rng.permutation(K)[:T]
    k = np.zeros((1, T, 1, K), np.float32)
    k[0, np.arange(T), 0, perm] = 1.0
    q = rng.normal(0, 1, (1, T, 1, K)).astype(np.float32)
    v = rng.normal(0, 1, (1, T, 1, V)).astype(np.float32)
    g = (-rng.uniform(0, 0.5, (1, T, 1))).astype(np.float32)
    beta = rng.uniform(0.1, 1, (1, T, 1)).astype(np.float32)
    for gate in (g, np.zeros_like(g)):
        o, fin = oracle.recurrent(q, k, v, gate, beta, scale=1.3)
        G = np.cumsum(gate[0, :, 0].astype(np.float64))
        kk, qq, vv = (x[0, :, 0].astype(np.float64) for x in (k, q, v))
        bb = beta[0, :, 0].astype(np.float64)
        for t in range(T):
            w = np.exp(G[t] - G[:t + 1]) * bb[:t + 1] * (kk[:t + 1] @ qq[t])
            np.testing.assert_allclose(o[0, t, 0], 1.3 * w @ vv[:t + 1], rtol=1e-12, atol=1e-13)
        S = sum(math.exp(G[-1] - G[j]) * bb[j] * np.outer(kk[j], vv[j]) for j in range(T))
        np.testing.assert_allclose(fin[0, 0], S, rtol=1e-12, atol=1e-13)


def test_unit_key_full_write_recalls_value():
    """beta = 1 with a unit-norm key overwrites exactly what the key reads:
    S_t^T k_t = v_t whatever the previous state and decay; reading with
    q_t = k_t and scale 1 returns v_t."""
    rng = np.random.default_rng(4)
    T, K, V = 20, 8, 5
    k = rng.normal(0, 1, (1, T, 1, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    k = k.astype(np.float32)
    v = rng.normal(0, 1, (1, T, 1, V)).astype(np.float32)
    g = (-rng.uniform(0, 1, (1, T, 1))).astype(np.float32)
    beta = np.ones((1, T, 1), np.float32)
    S0 = rng.normal(0, 1, (1, 1, K, V)).astype(np.float32)
    o, _ = oracle.recurrent(k, k, v, g, beta, scale=1.0, initial_state=S0)
    kn = k[0, :, 0].astype(np.float64)
    # float32 keys are unit norm only to ~1e-7; the recall error is of that order.
    np.testing.assert_allclose(o[0, :, 0] * 1.0, v[0, :, 0], rtol=0, atol=5e-6)
    assert np.all(np.abs(np.linalg.norm(kn, axis=1) - 1) < 1e-6)


def test_superposition():
    """For fixed q, k, g, beta the map (S0, v) -> (o, S) is linear."""
    rng = np.random.default_rng(5)
    T, K, V = 30, 8, 4
    q, k, v, g, beta = _rand_inputs(rng, 1, T, 1, 1, K, V)
    S0 = rng.normal(0, 1, (1, 1, K, V)).astype(np.float32)
    z = np.zeros_like
    o1, f1 = oracle.recurrent(q, k, v, g, beta, scale=1.0, use_l2norm=True, initial_state=S0)
    o2, f2 = oracle.recurrent(q, k, z(v), g, beta, scale=1.0, use_l2norm=True, initial_state=S0)
    o3, f3 = oracle.recurrent(q, k, v, g, beta, scale=1.0, use_l2norm=True, initial_state=None)
    np.testing.assert_allclose(o1, o2 + o3, rtol=0, atol=1e-12)
    np.testing.assert_allclose(f1, f2 + f3, rtol=0, atol=1e-12)
    o4, f4 = oracle.recurrent(q, k, 2 * v, g, beta, scale=1.0, use_l2norm=True)
    np.testing.assert_allclose(o4, 2 * o3, rtol=0, atol=1e-12)


def test_prefix_split_chains_state():
    """One call over tokens 1..T equals a call over 1..T1 followed by a call
    over T1+1..T started from the first call's final state."""
    rng = np.random.default_rng(6)
    T, T1, H, HV, K, V = 50, 17, 2, 4, 8, 8
    q, k, v, g, beta = _rand_inputs(rng, 1, T, H, HV, K, V)
    S0 = rng.normal(0, 0.1, (1, HV, K, V)).astype(np.float32)
    o, fin = oracle.recurrent(q, k, v, g, beta, use_l2norm=True, initial_state=S0)
    a = slice(0, T1)
    b = slice(T1, T)
    oa, fa = oracle.recurrent(q[:, a], k[:, a], v[:, a], g[:, a], beta[:, a], use_l2norm=True,
                              initial_state=S0)
    ob, fb = oracle.recurrent(q[:, b], k[:, b], v[:, b], g[:, b], beta[:, b], use_l2norm=True,
                              initial_state=fa.astype(np.float32))
    np.testing.assert_allclose(o[:, a], oa, rtol=0, atol=1e-14)
    # the handover state passes through float32 once, hence the looser bound
    np.testing.assert_allclose(o[:, b], ob, rtol=0, atol=1e-6)
    np.testing.assert_allclose(fin, fb, rtol=0, atol=1e-6)


def test_varlen_equals_separate_runs():
    rng = np.random.default_rng(7)
    lens = [5, 64, 1, 0, 70, 33]
    H, HV, K, V = 1, 2, 8, 4
    T = sum(lens)
    q, k, v, g, beta = _rand_inputs(rng, 1, T, H, HV, K, V)
    S0 = rng.normal(0, 0.1, (len(lens), HV, K, V)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, fin = oracle.recurrent(q, k, v, g, beta, use_l2norm=True, initial_state=S0, cu_seqlens=cu)
    for n, L in enumerate(lens):
        s = slice(cu[n], cu[n + 1])
        on, fn = oracle.recurrent(q[:, s], k[:, s], v[:, s], g[:, s], beta[:, s], use_l2norm=True,
                                  initial_state=S0[n:n + 1])
        np.testing.assert_array_equal(o[:, s], on)
        np.testing.assert_array_equal(fin[n:n + 1], fn)
    # an empty sequence hands its initial state straight through
    np.testing.assert_array_equal(fin[3], S0[3].astype(np.float64))


def test_grouped_value_heads_equal_repeated_key_heads():
    """Value head j reads key head j // (HV/H): contiguous groups.  Repeating
    each key head G times (repeat_interleave) and running with H' = HV must
    give the same result."""
    rng = np.random.default_rng(8)
    T, H, HV, K, V = 40, 2, 6, 8, 4
    q, k, v, g, beta = _rand_inputs(rng, 2, T, H, HV, K, V)
    o, fin = oracle.recurrent(q, k, v, g, beta, use_l2norm=True)
    G = HV // H
    qr, kr = (np.repeat(x, G, axis=2) for x in (q, k))
    o2, fin2 = oracle.recurrent(qr, kr, v, g, beta, use_l2norm=True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(fin, fin2)


def test_l2norm_scale_invariance():
    rng = np.random.default_rng(9)
    T, K, V = 25, 16, 8
    q, k, v, g, beta = _rand_inputs(rng, 1, T, 1, 1, K, V)
    c = rng.uniform(0.5, 4.0, (1, T, 1, 1)).astype(np.float32)
    c = (2.0 ** np.round(np.log2(c))).astype(np.float32)   # powers of two: exact scaling
    o1, f1 = oracle.recurrent(q, k, v, g, beta, use_l2norm=True)
    o2, f2 = oracle.recurrent(q * c, k * c[..., ::-1, :, :], v, g, beta, use_l2norm=True)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-6)
    np.testing.assert_allclose(f1, f2, rtol=0, atol=1e-6)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
@pytest.mark.parametrize("C", [1, 16, 64, None])
def test_chunked_form_matches_recurrence(T, C):
    rng = np.random.default_rng(10 + T)
    K, V = 16, 12
    q, k, v, g, beta = _rand_inputs(rng, 1, T, 1, 1, K, V, gmax=0.2)
    S0 = rng.normal(0, 0.3, (1, 1, K, V)).astype(np.float32)
    o, fin = oracle.recurrent(q, k, v, g, beta, scale=0.25, use_l2norm=True, initial_state=S0)
    oc, fc = chunked_unit(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], 0.25, True,
                          S0[0, 0], C=C or T)
    np.testing.assert_allclose(oc, o[0, :, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(fc, fin[0, 0], rtol=0, atol=1e-12)


def test_oracle_rejects_bad_arguments():
    rng = np.random.default_rng(11)
    q, k, v, g, beta = _rand_inputs(rng, 1, 4, 2, 3, 4, 4)   # HV % H != 0
    with pytest.raises(ValueError):
        oracle.recurrent(q, k, v, g, beta)
    q, k, v, g, beta = _rand_inputs(rng, 2, 4, 1, 1, 4, 4)
    with pytest.raises(ValueError):   # cu_seqlens with B > 1
        oracle.recurrent(q, k, v, g, beta, cu_seqlens=np.array([0, 4], np.int32))
