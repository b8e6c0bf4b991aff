"""Oracle for the gated delta rule forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never does, and the two
share no code: the only thing both sides use is the seeded input generator in
``workloads.py``, which holds none of the method's arithmetic.

Two implementations live here:

* ``recurrent`` -- the definition: the token-by-token recurrence in double
  precision, written in plain C (``gdn_oracle.c``), OpenMP over
  (sequence, value head) units.  See that file for the equations and where
  they come from.
* ``chunked.chunked_unit`` -- the 64-token chunked (WY) form in numpy float64,
  one unit at a time, exposing the per-chunk intermediates.  It reaches the
  same result up to rounding order and is used to check the recurrence and to
  debug.
* ``gating`` -- g and beta from A_log, dt_bias, a, b in float64 (``gating.py``),
  and ``recurrent_gated``, the recurrence fed with those gates rounded to
  float32 (the gates' type on the page that defines them); ``gating_bwd``, the
  gradients of the gate inputs given those of g and beta.

Parity is pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_*.py``
(hand-derived worked example, closed forms, invariants, the matrix-product
form of the recurrence, the chunked form).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compiles the C oracle with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        f = lib.gdn_oracle_forward
        P = ctypes.c_void_p
        f.argtypes = [P, P, P, P, P, P, P,
                      ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                      ctypes.c_double, ctypes.c_int,
                      P, ctypes.c_int64, P, P, P, ctypes.c_int]
        f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(x):
    """Exact float32 numpy view of a tensor/array (bf16 and fp32 convert exactly)."""
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float32).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def recurrent(q, k, v, g, beta, scale=None, use_l2norm=False, initial_state=None,
              cu_seqlens=None, units=None, nthreads=0):
    """Reference forward pass by the token recurrence, in float64.

    Arguments follow the GPU entry point: q, k [B,T,H,K]; v [B,T,HV,V];
    g, beta [B,T,HV]; initial_state [N,HV,K,V] or None; cu_seqlens [N+1] or
    None (then N = B and every batch row is one sequence of length T; else
    B must be 1).  ``units`` selects (sequence, value head) pairs as
    n*HV + j (default: all).

    Returns ``(o, final)``.  With ``units=None``: o is [B,T,HV,V] and final
    [N,HV,K,V] (float64).  With units: o is a list of [len_n, V] arrays and
    final is [len(units), K, V].
    """
    qf, kf, vf, gf, bf = (_f32(x) for x in (q, k, v, g, beta))
    B, T, H, K = qf.shape
    HV, V = vf.shape[2], vf.shape[3]
    if kf.shape != qf.shape or vf.shape[:2] != (B, T) or gf.shape != (B, T, HV) or bf.shape != (B, T, HV):
        raise ValueError("shape mismatch")
    if cu_seqlens is None:
        N = B
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("cu_seqlens requires B == 1")
        cu = np.asarray(_f32(cu_seqlens) if not isinstance(cu_seqlens, np.ndarray) else cu_seqlens)
        cu = np.ascontiguousarray(cu.astype(np.int64))
        N = cu.shape[0] - 1
    s0 = _f32(initial_state)
    if s0 is not None and s0.shape != (N, HV, K, V):
        raise ValueError("initial_state must be [N,HV,K,V]")
    if scale is None:
        scale = K ** -0.5
    all_units = units is None
    u = np.arange(N * HV, dtype=np.int64) if all_units else np.ascontiguousarray(np.asarray(units, dtype=np.int64))
    lens = cu[1:] - cu[:-1]
    ul = lens[u // HV]
    out_row = np.zeros(len(u), dtype=np.int64)
    if len(u) > 1:
        out_row[1:] = np.cumsum(ul)[:-1]
    out = np.zeros((int(ul.sum()), V), dtype=np.float64)
    fin = np.zeros((len(u), K, V), dtype=np.float64)
    lib = _load()
    rc = lib.gdn_oracle_forward(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(gf), _ptr(bf), _ptr(s0), _ptr(cu),
                                N, H, HV, K, V, float(scale), int(bool(use_l2norm)),
                                _ptr(u), len(u), _ptr(out_row), _ptr(out), _ptr(fin), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    if not all_units:
        return [out[out_row[i]:out_row[i] + ul[i]] for i in range(len(u))], fin
    o = np.zeros((B * T, HV, V), dtype=np.float64)
    for i, uu in enumerate(u):
        n, j = divmod(int(uu), HV)
        o[cu[n]:cu[n + 1], j, :] = out[out_row[i]:out_row[i] + ul[i]]
    return o.reshape(B, T, HV, V), fin.reshape(N, HV, K, V)


from .gating import gating, gating_bwd, sigmoid, softplus  # noqa: E402


def recurrent_gated(q, k, v, A_log, dt_bias, a, b, **kw):
    """``recurrent`` with g and beta computed from the raw gate inputs: a, b
    [B,T,HV] (or [N,HV] rows of one step each when q is [N,1,H,K]), A_log,
    dt_bias [HV].  The gates are rounded to float32 before the recurrence, as
    the gating operator returns them."""
    g, beta = gating(A_log, dt_bias, a, b)
    return recurrent(q, k, v, g.astype(np.float32), beta.astype(np.float32), **kw)


def add_gates(x):
    """Adds g and beta (float32 tensors on the device of x["a"]) computed from
    the raw gate inputs of an input dict of ``workloads`` -- the un-fused
    entry points take them as inputs.  Returns x."""
    import torch
    g, beta = gating(x["A_log"], x["dt_bias"], x["a"], x["b"])
    dev = x["a"].device
    x["g"] = torch.from_numpy(g.astype(np.float32)).to(dev)
    x["beta"] = torch.from_numpy(beta.astype(np.float32)).to(dev)
    return x


def recurrent_pool(q, k, v, g, beta, pool, indices, read_initial=True, **kw):
    """``recurrent`` against a state pool [P,HV,K,V] (any float type): sequence
    n starts from pool[indices[n]] (from zero when read_initial is false or the
    slot lies outside [0, P), a sequence with no state) and its final state
    replaces that slot.  Returns (o, pool_after) with pool_after a float64 copy
    of the pool holding the final states (unrounded) in the named slots."""
    import torch
    pool64 = pool.detach().to("cpu", torch.float64).numpy() if isinstance(pool, torch.Tensor) \
        else np.asarray(pool, dtype=np.float64)
    idx = np.asarray(indices.cpu() if isinstance(indices, torch.Tensor) else indices, dtype=np.int64)
    P = pool64.shape[0]
    valid = (idx >= 0) & (idx < P)
    s0 = np.zeros((len(idx),) + pool64.shape[1:], dtype=np.float64)
    if read_initial:
        s0[valid] = pool64[idx[valid]]
    o, fin = recurrent(q, k, v, g, beta, initial_state=s0.astype(np.float32), **kw)
    after = pool64.copy()
    after[idx[valid]] = fin[valid]
    return o, after
