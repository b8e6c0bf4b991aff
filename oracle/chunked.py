"""Chunked (WY) form of the gated delta rule, float64 numpy -- TEST INFRASTRUCTURE ONLY.

This follows the six steps that the page "NPU Training Operators - GDN" lists in
its operator-semantics section for the chunked algorithm (chunk-local gate
cumsum, the gated beta*K*K^T product inside a chunk, the lower-triangular
solve, recomputing w/u, the inter-chunk state recurrence, the output readout),
which the page "[Qwen3.5][Feature] support fla triton kernel for qwen3.5"
(FastDeploy PR #7024) names as the prefill algorithm in its Motivation section
and splits into files in its file table (chunk size 64 per the NPU page's
tiling section).  The pages do not print the equations; the ones below are
derived from the recurrence (see gdn_oracle.c) and are the same mathematics,
up to rounding order.

One unit = one sequence and one value head.  Per chunk of L <= C rows, with
gamma the inclusive cumsum of g inside the chunk, r / rho the L2-norm factors of
k / q (1 when the norm is off), h the state at the chunk start (K x V):

  A[i,j]  = beta_i r_i r_j exp(gamma_i - gamma_j) (k_i . k_j)   for i > j, else 0
  T       = (I + A)^-1
  W       = T diag(beta_i exp(gamma_i) r_i) K
  U       = T diag(beta_i) V
  V_new   = U - W h
  h_next  = exp(gamma_L) h + K^T diag(r_j exp(gamma_L - gamma_j)) V_new
  O       = scale ( diag(rho_i exp(gamma_i)) Q h
                    + (M * [rho_i r_j exp(gamma_i - gamma_j)] * Q K^T) V_new )
            with M[i,j] = [j <= i]

The exponentials only ever take gamma_i - gamma_j with i >= j (never positive
for g <= 0) and gamma itself, as the safe_exp helper in that PR's file table
implies (mask first, then exponentiate).
"""
from __future__ import annotations

import numpy as np


def _norm_factor(x, use_l2norm):
    if not use_l2norm:
        return np.ones(x.shape[0])
    return 1.0 / np.sqrt(np.sum(x * x, axis=1) + 1e-6)


def chunked_unit(q, k, v, g, beta, scale, use_l2norm, S0=None, C=64, keep=False):
    """Runs one (sequence, value head) unit through the chunked form.

    q, k: [L, K]; v: [L, V]; g, beta: [L]; S0: [K, V] or None.
    Returns (o [L, V], final [K, V]) and, with keep=True, a list with one dict
    of intermediates (gamma, A, T, W, U, h, v_new) per chunk.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    Lt, K = k.shape
    V = v.shape[1]
    h = np.zeros((K, V)) if S0 is None else np.array(S0, np.float64)
    rho = _norm_factor(q, use_l2norm)
    r = _norm_factor(k, use_l2norm)
    o = np.zeros((Lt, V))
    trace = []
    for c0 in range(0, Lt, C):
        sl = slice(c0, min(c0 + C, Lt))
        Kc, Qc, Vc = k[sl], q[sl], v[sl]
        bc, rc, pc = beta[sl], r[sl], rho[sl]
        gam = np.cumsum(g[sl])
        L = Kc.shape[0]
        diff = gam[:, None] - gam[None, :]
        lower = np.tril(np.ones((L, L), dtype=bool), -1)
        causal = np.tril(np.ones((L, L), dtype=bool), 0)
        dec = np.zeros((L, L))
        dec[causal] = np.exp(diff[causal])
        A = np.where(lower, (bc * rc)[:, None] * rc[None, :] * dec * (Kc @ Kc.T), 0.0)
        T = np.linalg.inv(np.eye(L) + A)
        W = T @ ((bc * np.exp(gam) * rc)[:, None] * Kc)
        U = T @ (bc[:, None] * Vc)
        v_new = U - W @ h
        P = np.where(causal, pc[:, None] * rc[None, :] * dec * (Qc @ Kc.T), 0.0)
        o[sl] = scale * ((pc * np.exp(gam))[:, None] * (Qc @ h) + P @ v_new)
        if keep:
            trace.append(dict(gamma=gam, A=A, T=T, W=W, U=U, h=h.copy(), v_new=v_new))
        gL = gam[-1]
        h = np.exp(gL) * h + Kc.T @ ((rc * np.exp(gL - gam))[:, None] * v_new)
    if keep:
        return o, h, trace
    return o, h
