"""Gradients of the gated delta rule forward pass, float64 -- TEST INFRASTRUCTURE ONLY.

Only ``tests/`` and the ``cpu_baseline`` leg of ``bench.py`` may use this
module; the GPU library never does and shares no code with it.

What it computes: the reverse-mode derivative of the token recurrence that
``gdn_oracle.c`` runs forward (the recurrence of the Gated Delta Networks paper
that the page "NPU Training Operators - GDN" cites in its operator-semantics
section; that page lists the backward operators dq, dk, dv, d(beta), dg and
the initial-state gradient beside the forward ones).  For one (sequence, value
head) unit, the forward step at token t is, with kh/qh the (optionally
L2-normalised) key/query rows and a = exp(g_t):

    P   = a S_{t-1}                 (forget)
    u   = P^T kh
    d   = beta_t (v_t - u)          (delta-rule error)
    S_t = P + kh d^T                (write)
    o_t = scale S_t^T qh            (read)

Given do_t for every token and dS_T (the gradient of the final state, zero
when no final state is used), walking t = T..1 applies the chain rule to those
five lines in reverse order:

    dS    += scale qh do_t^T ;   dqh = scale S_t do_t
    dkh    = dS d ;             dd  = dS^T kh          (from the write)
    dv_t   = beta_t dd ;        dbeta_t = dd . (v_t - u) ;   du = -beta_t dd
    dP     = dS + kh du^T ;     dkh += P du            (from u = P^T kh)
    dg_t   = <dP, P> ;          dS   = a dP            (from the forget step)

and at the end dS is the gradient of the initial state.  With the L2 norm,
x_hat = x / sqrt(|x|^2 + 1e-6), so dx = f (dx_hat - x_hat (x_hat . dx_hat))
with f = 1/sqrt(|x|^2 + 1e-6).  A key head's gradient sums the contributions of
the value heads that share it.

``forward64`` runs the same forward recurrence in numpy float64 without
rounding its inputs to float32; the finite-difference pins of the backward are
taken on it (and it is itself checked against the C oracle).

Cost: O(T K V) per unit in numpy per token, for small cases only.
"""
from __future__ import annotations

import numpy as np


def _as64(x):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _seq_bounds(B, T, cu_seqlens):
    if cu_seqlens is None:
        return [(b * T, (b + 1) * T) for b in range(B)]
    if B != 1:
        raise ValueError("cu_seqlens requires B == 1")
    cu = [int(c) for c in np.asarray(_as64(cu_seqlens)).tolist()]
    return [(cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def _normed(x, use_l2norm):
    if not use_l2norm:
        return x.copy(), 1.0
    f = 1.0 / np.sqrt(np.dot(x, x) + 1e-6)
    return x * f, f


def forward64(q, k, v, g, beta, scale=None, use_l2norm=False, initial_state=None, cu_seqlens=None):
    """The forward recurrence in float64 on float64 inputs.  Shapes as in
    ``oracle.recurrent``.  Returns (o [B,T,HV,V], final [N,HV,K,V])."""
    q, k, v, g, beta = (_as64(x) for x in (q, k, v, g, beta))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    G = HV // H
    if scale is None:
        scale = K ** -0.5
    seqs = _seq_bounds(B, T, cu_seqlens)
    s0 = _as64(initial_state)
    qf, kf = q.reshape(B * T, H, K), k.reshape(B * T, H, K)
    vf, gf, bf = v.reshape(B * T, HV, V), g.reshape(B * T, HV), beta.reshape(B * T, HV)
    o = np.zeros((B * T, HV, V))
    fin = np.zeros((len(seqs), HV, K, V))
    for n, (t0, t1) in enumerate(seqs):
        for j in range(HV):
            jk = j // G
            S = np.zeros((K, V)) if s0 is None else s0[n, j].copy()
            for t in range(t0, t1):
                qh, _ = _normed(qf[t, jk], use_l2norm)
                kh, _ = _normed(kf[t, jk], use_l2norm)
                S = np.exp(gf[t, j]) * S
                d = bf[t, j] * (vf[t, j] - S.T @ kh)
                S = S + np.outer(kh, d)
                o[t, j] = scale * (S.T @ qh)
            fin[n, j] = S
    return o.reshape(B, T, HV, V), fin


def backward(q, k, v, g, beta, do, dht=None, scale=None, use_l2norm=False, initial_state=None,
             cu_seqlens=None):
    """Gradients of the forward pass (o and the final state) with respect to
    its inputs.

    q, k [B,T,H,K]; v, do [B,T,HV,V]; g, beta [B,T,HV]; dht (gradient of the
    final state) and initial_state [N,HV,K,V] or None.  Returns a dict with
    dq, dk [B,T,H,K], dv [B,T,HV,V], dg, dbeta [B,T,HV] and dh0 [N,HV,K,V]
    (float64).
    """
    q, k, v, g, beta, do = (_as64(x) for x in (q, k, v, g, beta, do))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    G = HV // H
    if scale is None:
        scale = K ** -0.5
    seqs = _seq_bounds(B, T, cu_seqlens)
    s0, dS_end = _as64(initial_state), _as64(dht)
    qf, kf = q.reshape(B * T, H, K), k.reshape(B * T, H, K)
    vf, gf, bf = v.reshape(B * T, HV, V), g.reshape(B * T, HV), beta.reshape(B * T, HV)
    dof = do.reshape(B * T, HV, V)
    dq, dk = np.zeros_like(qf), np.zeros_like(kf)
    dv, dg, db = np.zeros_like(vf), np.zeros_like(gf), np.zeros_like(bf)
    dh0 = np.zeros((len(seqs), HV, K, V))
    for n, (t0, t1) in enumerate(seqs):
        for j in range(HV):
            jk = j // G
            # forward, keeping every state S_{t-1} and S_t
            S = np.zeros((K, V)) if s0 is None else s0[n, j].copy()
            states = [S]
            for t in range(t0, t1):
                kh, _ = _normed(kf[t, jk], use_l2norm)
                P = np.exp(gf[t, j]) * S
                d = bf[t, j] * (vf[t, j] - P.T @ kh)
                S = P + np.outer(kh, d)
                states.append(S)
            dS = np.zeros((K, V)) if dS_end is None else dS_end[n, j].copy()
            for t in range(t1 - 1, t0 - 1, -1):
                i = t - t0
                S_prev, S_t = states[i], states[i + 1]
                qh, fq = _normed(qf[t, jk], use_l2norm)
                kh, fk = _normed(kf[t, jk], use_l2norm)
                a, bt = np.exp(gf[t, j]), bf[t, j]
                P = a * S_prev
                u = P.T @ kh
                d = bt * (vf[t, j] - u)
                # read: o_t = scale S_t^T qh
                dS = dS + scale * np.outer(qh, dof[t, j])
                dqh = scale * (S_t @ dof[t, j])
                # write: S_t = P + kh d^T
                dkh = dS @ d
                dd = dS.T @ kh
                # error: d = beta (v - u)
                dv[t, j] = bt * dd
                db[t, j] = dd @ (vf[t, j] - u)
                du = -bt * dd
                # u = P^T kh
                dP = dS + np.outer(kh, du)
                dkh = dkh + P @ du
                # forget: P = exp(g) S_prev
                dg[t, j] = np.sum(dP * P)
                dS = a * dP
                if use_l2norm:
                    dqh = fq * (dqh - qh * (qh @ dqh))
                    dkh = fk * (dkh - kh * (kh @ dkh))
                dq[t, jk] += dqh
                dk[t, jk] += dkh
            dh0[n, j] = dS
    return {"dq": dq.reshape(B, T, H, K), "dk": dk.reshape(B, T, H, K), "dv": dv.reshape(B, T, HV, V),
            "dg": dg.reshape(B, T, HV), "dbeta": db.reshape(B, T, HV), "dh0": dh0}
