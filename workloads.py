"""Seeded synthetic inputs for the chunked gated delta rule.

This module is shared by the oracle-side tests and the GPU-side tests and
benchmark.  It holds none of the method's arithmetic: it only draws random
tensors.  The gates are drawn as their raw inputs (a, b per token and value
head, A_log and dt_bias per value head); g and beta follow from them by the
gating law (g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b), the
fused gating operator of the page "[Qwen3.5][Feature] support fla triton
kernel for qwen3.5" (FastDeploy PR #7024), "Usage or Command", item 5), which
each side computes itself: the oracle in float64, the GPU path in its kernels.

Draw order (one torch.Generator on the target device, seeded): q, k, v, a, b,
A_log, dt_bias, initial_state, then (only when qk_common is set) the shared
key-head directions; packed workloads first draw their sequence lengths from a
separate CPU generator with the same seed.  (CPU and GPU
generators produce different streams: a workload drawn on the GPU has the same
shapes and lengths as on the CPU but other values.)  q/k/v and a/b are drawn
in float32 and rounded to bfloat16 (round to nearest even), the type a model's
projections produce; the float32 check mode uses those same bf16-representable
values stored as float32, so one oracle run serves both.
"N(0, s)" below means standard deviation s.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int                 # per-sequence length (equal-length) or 0 for varlen
    H: int
    HV: int
    K: int
    V: int
    use_l2norm: bool = True
    scale: Optional[float] = None          # None -> 1/sqrt(K)
    a_log_hi: float = math.log(16.0)      # A_log ~ U(0, a_log_hi)
    b_std: float = 1.0                     # b ~ N(b_mean, b_std)
    b_mean: float = 0.0
    a_mean: float = 0.0                    # a ~ N(a_mean, 1)
    qk_std: float = 1.0                    # q, k ~ N(0, qk_std)
    qk_common: float = 0.0                 # q, k += qk_common * c_h, c_h ~ N(0, qk_std) per key head
    init: str = "none"                     # "none" | "all" | "odd"
    init_std: float = 0.05
    n_seqs: int = 0                        # varlen: number of sequences
    max_len: int = 0                       # varlen: lengths ~ U{min_len..max_len}
    min_len: int = 1
    lengths: Optional[tuple] = None        # varlen: explicit lengths (overrides the draw)

    @property
    def varlen(self) -> bool:
        return self.n_seqs > 0

    @property
    def eff_scale(self) -> float:
        return self.scale if self.scale is not None else self.K ** -0.5


# The five workloads the throughput metric and the parity suite are quoted on.
WORKLOADS = {
    # Tiny check: B=1, T=256, H=HV=2, K=V=64, L2 norm on, no initial state.
    "tiny": Workload("tiny", B=1, T=256, H=2, HV=2, K=64, V=64),
    # Equal-length GVA prefill: B=4, T=4096, H=16, HV=32, K=V=128, initial state.
    "gva": Workload("gva", B=4, T=4096, H=16, HV=32, K=128, V=128, init="all"),
    # Varlen packed prefill: 64 sequences, lengths ~ U{1..2048}, initial state on odd ones.
    "varlen": Workload("varlen", B=1, T=0, H=16, HV=32, K=128, V=128, init="odd",
                       n_seqs=64, max_len=2048),
    # Long-context single sequence: T=131072, slow decay A_log ~ U(0, ln 4).
    "long": Workload("long", B=1, T=131072, H=16, HV=32, K=128, V=128,
                     a_log_hi=math.log(4.0)),
    # Wide large-batch prefill: B=16, T=16384, H=32, HV=64, no L2 norm,
    # scale 1/sqrt(128), b ~ N(0, 2), initial state.
    "wide": Workload("wide", B=16, T=16384, H=32, HV=64, K=128, V=128, use_l2norm=False,
                     scale=128 ** -0.5, b_std=2.0, init="all"),
}

# The wide workload as literally specified diverges (no L2 norm with q,k ~ N(0,1)
# at K=128 gives |k|^2 ~ 128, so the erase factor 1 - beta*|k|^2 is ~ -100).
# Its parity counterpart keeps every shape, flag, scale and gate law but draws
# q, k ~ N(0, 1/sqrt(K)), i.e. |k|^2 ~ 1.
WORKLOADS["wide_stable"] = dataclasses.replace(WORKLOADS["wide"], name="wide_stable",
                                               qk_std=128 ** -0.5)


def scaled(w: Workload, name: str, **kw) -> Workload:
    """A smaller variant of a workload with the same distributions."""
    return dataclasses.replace(w, name=name, **kw)


def make_inputs(w: Workload, seed: int = 0, device="cpu", io_dtype=torch.bfloat16):
    """Draws one batch of inputs for workload ``w``.

    Returns a dict with q, k [B,T,H,K], v [B,T,HV,V] and the raw gate inputs
    a, b [B,T,HV] in ``io_dtype`` (bf16 values; float32 holds the same
    values), A_log, dt_bias [HV] float32, initial_state [N,HV,K,V] float32 or
    None, cu_seqlens [N+1] int32 or None, scale, use_l2norm, and the sequence
    lengths as a Python list.
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    f32 = torch.float32
    if w.varlen:
        if w.lengths is not None:
            lens = list(w.lengths)
        else:
            # lengths come from a CPU generator of their own, so that a packed
            # workload has the same sequence lengths whichever device draws the values
            lgen = torch.Generator()
            lgen.manual_seed(seed)
            lens = torch.randint(w.min_len, w.max_len + 1, (w.n_seqs,), generator=lgen).tolist()
        N = len(lens)
        B, T = 1, int(sum(lens))
        cu = torch.zeros(N + 1, dtype=torch.int32)
        if N:
            cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
        cu = cu.to(dev)
    else:
        N, B, T = w.B, w.B, w.T
        lens = [T] * B
        cu = None
    H, HV, K, V = w.H, w.HV, w.K, w.V

    def randn(*shape, std=1.0):
        return torch.randn(*shape, generator=gen, device=dev, dtype=f32) * std

    def io(x):
        return x.to(torch.bfloat16).to(io_dtype)

    q = randn(B, T, H, K, std=w.qk_std)
    k = randn(B, T, H, K, std=w.qk_std)
    v = io(randn(B, T, HV, V))
    a = io(randn(B, T, HV) + w.a_mean)
    b = io(randn(B, T, HV, std=w.b_std) + w.b_mean)
    a_log = torch.rand(HV, generator=gen, device=dev, dtype=f32) * w.a_log_hi
    dt_bias = torch.rand(HV, generator=gen, device=dev, dtype=f32)
    if w.init == "none":
        s0 = None
    else:
        s0 = randn(N, HV, K, V, std=w.init_std)
        if w.init == "odd":
            s0[0::2] = 0.0
    if w.qk_common:
        # keys and queries of one key head share a direction: neighbouring keys
        # overlap, so the delta rule's erase term is large
        c = randn(1, 1, H, K, std=w.qk_std) * w.qk_common
        q, k = q + c, k + c
    q, k = io(q), io(k)
    return dict(q=q, k=k, v=v, a=a, b=b, A_log=a_log, dt_bias=dt_bias, initial_state=s0,
                cu_seqlens=cu, scale=w.eff_scale, use_l2norm=w.use_l2norm, lens=lens,
                N=N, workload=w)


def make_grad_inputs(x, seed: int = 1, dht_std: float = 0.1):
    """Draws the output gradients of a backward pass for the forward inputs
    ``x`` of ``make_inputs``: do with v's shape, dtype and device (N(0, 1)
    values rounded to bf16) and dht [N,HV,K,V] float32 ~ N(0, dht_std^2).
    Adds them to x as x["do"], x["dht"] and returns x."""
    v = x["v"]
    dev = v.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    w = x["workload"]
    do = torch.randn(*v.shape, generator=gen, device=dev, dtype=torch.float32)
    x["do"] = do.to(torch.bfloat16).to(v.dtype)
    x["dht"] = torch.randn(x["N"], w.HV, w.K, w.V, generator=gen, device=dev, dtype=torch.float32) * dht_std
    return x


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One decode step: N sequences, one token each, states in a pool."""
    name: str
    N: int
    H: int
    HV: int
    K: int
    V: int
    pool_size: int
    n_pad: int = 0                 # rows marked -1 (padding)
    use_l2norm: bool = True
    scale: Optional[float] = None
    a_log_hi: float = math.log(16.0)
    state_std: float = 0.05
    pool_dtype: torch.dtype = torch.float32

    @property
    def eff_scale(self) -> float:
        return self.scale if self.scale is not None else self.K ** -0.5


# A serving-style decode batch of the GVA model shape: 256 running sequences in
# a 512-slot state pool, 8 padded rows; the same with a bf16 pool.
DECODE_WORKLOADS = {
    "decode": DecodeWorkload("decode", N=256, H=16, HV=32, K=128, V=128, pool_size=512, n_pad=8),
    "decode_bf16pool": DecodeWorkload("decode_bf16pool", N=256, H=16, HV=32, K=128, V=128, pool_size=512,
                                      n_pad=8, pool_dtype=torch.bfloat16),
}


def make_decode_inputs(w: DecodeWorkload, seed: int = 0, device="cpu", io_dtype=torch.bfloat16):
    """Draws one decode step: q, k [N,H,K], v [N,HV,V] and the raw gate inputs
    a, b [N,HV] (bf16 values), A_log, dt_bias [HV] float32, a state pool [P,HV,K,V]
    of w.pool_dtype ~ N(0, state_std) and int32 slot indices (a random injective map into the
    pool, the first n_pad rows set to -1).  Values come from a generator on
    ``device``; the indices from a CPU generator of their own."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    f32 = torch.float32

    def randn(*shape, std=1.0):
        return torch.randn(*shape, generator=gen, device=dev, dtype=f32) * std

    def io(x):
        return x.to(torch.bfloat16).to(io_dtype)

    N, H, HV, K, V = w.N, w.H, w.HV, w.K, w.V
    q = io(randn(N, H, K))
    k = io(randn(N, H, K))
    v = io(randn(N, HV, V))
    a = io(randn(N, HV))
    b = io(randn(N, HV))
    a_log = torch.rand(HV, generator=gen, device=dev, dtype=f32) * w.a_log_hi
    dt_bias = torch.rand(HV, generator=gen, device=dev, dtype=f32)
    pool = randn(w.pool_size, HV, K, V, std=w.state_std).to(w.pool_dtype)
    igen = torch.Generator()
    igen.manual_seed(seed)
    idx = torch.randperm(w.pool_size, generator=igen)[:N].to(torch.int32)
    idx[: w.n_pad] = -1
    return dict(q=q, k=k, v=v, a=a, b=b, A_log=a_log, dt_bias=dt_bias, pool=pool, idx=idx.to(dev),
                scale=w.eff_scale, use_l2norm=w.use_l2norm, workload=w)
