"""Pins of the oracle's state-pool form (``oracle.recurrent_pool``): the pool
is plain indexing around the recurrence, so each pin ties it to the recurrence
with an explicit initial state (CPU only)."""
import numpy as np
import pytest
import torch

import oracle


def _case(N=4, T=9, H=1, HV=2, K=4, V=3, seed=0):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.normal(size=s).astype(np.float32)
    q, k = f(N, T, H, K), f(N, T, H, K)
    v = f(N, T, HV, V)
    g = -np.abs(f(N, T, HV)) * 0.3
    beta = rng.uniform(0.1, 0.9, size=(N, T, HV)).astype(np.float32)
    return q, k, v, g, beta


def test_identity_slots_equal_explicit_initial_state():
    q, k, v, g, beta = _case()
    pool = np.random.default_rng(1).normal(size=(4, 2, 4, 3)).astype(np.float32)
    o1, after = oracle.recurrent_pool(q, k, v, g, beta, pool, np.arange(4), use_l2norm=True)
    o2, fin = oracle.recurrent(q, k, v, g, beta, initial_state=pool, use_l2norm=True)
    assert np.array_equal(o1, o2) and np.array_equal(after, fin)


def test_permuted_slots_padding_and_untouched_slots():
    q, k, v, g, beta = _case(seed=2)
    pool = np.random.default_rng(3).normal(size=(7, 2, 4, 3)).astype(np.float32)
    idx = np.array([5, -1, 0, 9])          # a padding row (-1) and a slot past the pool
    o, after = oracle.recurrent_pool(q, k, v, g, beta, pool, idx, use_l2norm=True)
    s0 = np.zeros((4, 2, 4, 3), np.float32)
    s0[0], s0[2] = pool[5], pool[0]
    o_ref, fin = oracle.recurrent(q, k, v, g, beta, initial_state=s0, use_l2norm=True)
    assert np.array_equal(o, o_ref)
    assert np.array_equal(after[5], fin[0]) and np.array_equal(after[0], fin[2])
    for s in (1, 2, 3, 4, 6):               # slots no valid row names keep their values
        assert np.array_equal(after[s], pool[s].astype(np.float64))


def test_read_initial_false_starts_from_zero():
    q, k, v, g, beta = _case(seed=4)
    pool = np.random.default_rng(5).normal(size=(4, 2, 4, 3)).astype(np.float32)
    o, after = oracle.recurrent_pool(q, k, v, g, beta, pool, np.array([3, 2, 1, 0]), read_initial=False)
    o_ref, fin = oracle.recurrent(q, k, v, g, beta)
    assert np.array_equal(o, o_ref) and np.array_equal(after[[3, 2, 1, 0]], fin)


def test_bf16_pool_values_are_read_exactly():
    q, k, v, g, beta = _case(seed=6)
    pool = torch.randn(4, 2, 4, 3, generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    o, _ = oracle.recurrent_pool(q, k, v, g, beta, pool, np.arange(4))
    o_ref, _ = oracle.recurrent(q, k, v, g, beta, initial_state=pool.float().numpy())
    assert np.array_equal(o, o_ref)
