"""Gate computation of the gated delta rule, float64 -- TEST INFRASTRUCTURE ONLY.

The page "[Qwen3.5][Feature] support fla triton kernel for qwen3.5"
(FastDeploy PR #7024) defines the fused gating operator in its file table and in
"Usage or Command", item 5: per token and value head,

    g    = -exp(A_log) * softplus(a + dt_bias)
    beta = sigmoid(b)

with A_log and dt_bias one value per value head and a, b one value per (token,
value head); both results are float32 tensors on that page.  The page "gdn.py"
(LightLLM) passes the same four inputs (A_log, dt_bias, a_raw, b_raw) to its
decode kernel instead of g and beta, so the gating may also happen inside the
recurrence kernel.

softplus(x) = ln(1 + e^x) and sigmoid(x) = 1 / (1 + e^-x), the textbook
functions (the page states no threshold or approximation).  They are evaluated
here in the overflow-free forms max(x, 0) + log1p(exp(-|x|)) and, for
sigmoid, with the exponent taken of -|x|; both are exact rewrites.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def softplus(x):
    x = _f64(x)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    x = _f64(x)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gating(A_log, dt_bias, a, b):
    """g, beta in float64 for a, b [..., HV] and A_log, dt_bias [HV]."""
    A_log, dt_bias, a, b = (_f64(x) for x in (A_log, dt_bias, a, b))
    if A_log.shape != dt_bias.shape or A_log.ndim != 1 or a.shape != b.shape or a.shape[-1] != A_log.shape[0]:
        raise ValueError("gating expects A_log, dt_bias [HV] and a, b [..., HV]")
    g = -np.exp(A_log) * softplus(a + dt_bias)
    return g, sigmoid(b)


def gating_bwd(A_log, dt_bias, a, b, dg, dbeta):
    """Gradients of the gate inputs in float64, given dg and dbeta [..., HV]
    (the gradients of g and beta, as the chunked backward pass returns them).

    From the two definitions above, with x = a + dt_bias and the textbook
    derivatives softplus'(x) = sigmoid(x), sigmoid'(b) = sigmoid(b)(1 -
    sigmoid(b)), and d/dA_log exp(A_log) = exp(A_log):

        da       = dg * (-exp(A_log) * sigmoid(a + dt_bias))
        db       = dbeta * beta * (1 - beta)
        ddt_bias = sum of da over every axis but the head axis
        dA_log   = sum of dg * g over every axis but the head axis

    Returns da, db (shape of a), dA_log, ddt_bias [HV]."""
    A_log, dt_bias, a, b, dg, dbeta = (_f64(x) for x in (A_log, dt_bias, a, b, dg, dbeta))
    if dg.shape != a.shape or dbeta.shape != b.shape:
        raise ValueError("gating_bwd expects dg, dbeta shaped like a, b")
    g, beta = gating(A_log, dt_bias, a, b)
    da = dg * (-np.exp(A_log) * sigmoid(a + dt_bias))
    db = dbeta * beta * (1.0 - beta)
    HV = A_log.shape[0]
    dA_log = (dg * g).reshape(-1, HV).sum(axis=0)
    ddt_bias = da.reshape(-1, HV).sum(axis=0)
    return da, db, dA_log, ddt_bias
