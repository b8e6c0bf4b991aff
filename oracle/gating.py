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
