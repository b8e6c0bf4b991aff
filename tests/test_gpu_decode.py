"""GPU parity of the fused recurrent decode step (in-place, pool-indexed state)
against the fp64 oracle, through the C ABI.

The oracle runs the token recurrence for the valid rows, starting from their
pool slots.  Bars as for prefill: bf16 inputs -> 2e-2 on o and 1e-2 on the
updated state; fp32 check mode -> 1e-4 on both.  Padding rows (slot -1 or a
slot outside the pool) must leave their slot bit-identical and write zeros,
and slots no row names must stay bit-identical.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: (2e-2, 1e-2), torch.float32: (1e-4, 1e-4)}
DEV = torch.device("cuda:0")


def _gdn():
    import gated_deltanet_chunked_delta_amd as gdn
    gdn.load_library()
    return gdn


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def make_case(w, N, pool_size, pad_rows, seed=0):
    """Decode inputs for N rows (workload w's distributions, T = 1), a pool
    drawn N(0, 0.05) and slot indices: a random injective map of the rows to
    the pool, with the rows in pad_rows marked -1 (and the last of them, if
    any, pointed past the pool instead)."""
    x = oracle.add_gates(make_inputs(scaled(w, w.name + "_decode", B=N, T=1, init="none"), seed=seed))
    gen = torch.Generator().manual_seed(seed + 1)
    pool = torch.randn(pool_size, w.HV, w.K, w.V, generator=gen) * 0.05
    idx = torch.randperm(pool_size, generator=gen)[:N].to(torch.int32)
    for i, r in enumerate(pad_rows):
        idx[r] = pool_size + 3 if i == len(pad_rows) - 1 and len(pad_rows) > 1 else -1
    return x, pool, idx


def oracle_decode(x, pool, idx, steps=1):
    valid = [r for r in range(idx.numel()) if 0 <= int(idx[r]) < pool.shape[0]]
    sel = torch.tensor(valid, dtype=torch.long)
    s0 = pool[idx[sel].long()].double()
    o, fin = oracle.recurrent(x["q"][sel], x["k"][sel], x["v"][sel], x["g"][sel], x["beta"][sel],
                              scale=x["scale"], use_l2norm=x["use_l2norm"], initial_state=s0)
    return valid, o, fin


def run_decode(x, pool, idx, dtype, t=0):
    gdn = _gdn()
    pool_d = pool.to(DEV).contiguous()
    o = gdn.fused_recurrent_gated_delta_rule_update(
        x["q"][:, t].to(DEV, dtype), x["k"][:, t].to(DEV, dtype), x["v"][:, t].to(DEV, dtype),
        x["g"][:, t].to(DEV), x["beta"][:, t].to(DEV), pool_d, idx.to(DEV), scale=x["scale"],
        use_qk_l2norm_in_kernel=x["use_l2norm"])
    torch.cuda.synchronize()
    return o.float().cpu(), pool_d.cpu()


def check(x, pool, idx, dtype):
    o, pool_after = run_decode(x, pool, idx, dtype)
    valid, o_ref, f_ref = oracle_decode(x, pool, idx)
    to, tf = TOL[dtype]
    eo = float(np.abs(o[valid].numpy().astype(np.float64) - o_ref[:, 0]).max())
    slots = idx[valid].long()
    ef = float(np.abs(pool_after[slots].numpy().astype(np.float64) - f_ref).max())
    _say(f"    max|do|={eo:.3e} (bar {to})  max|dS|={ef:.3e} (bar {tf})")
    assert eo <= to and ef <= tf
    pads = [r for r in range(idx.numel()) if r not in valid]
    assert torch.all(o[pads] == 0)
    untouched = torch.ones(pool.shape[0], dtype=torch.bool)
    untouched[slots] = False
    assert torch.equal(pool_after[untouched], pool[untouched])


CASES = {
    "tiny": (WORKLOADS["tiny"], 7, 10, (2, 5)),
    "gva": (WORKLOADS["gva"], 48, 64, (0, 17, 47)),
    "k64_v128": (scaled(WORKLOADS["gva"], "k64_v128", H=2, HV=4, K=64, V=128), 9, 12, (3,)),
    "k128_v64": (scaled(WORKLOADS["gva"], "k128_v64", H=1, HV=3, K=128, V=64), 9, 9, ()),
    "no_l2norm": (scaled(WORKLOADS["wide_stable"], "wide_dec", H=2, HV=4), 16, 20, (1,)),
}


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("name", list(CASES))
def test_decode_parity(name, dtype):
    w, N, P, pads = CASES[name]
    _say(f"[decode] {name} dtype={dtype} N={N} pool={P} pads={pads}")
    x, pool, idx = make_case(w, N, P, pads)
    check(x, pool, idx, dtype)


def test_decode_steps_follow_the_recurrence():
    """Four decode steps on the same slots equal the oracle over four tokens."""
    gdn = _gdn()
    w = scaled(WORKLOADS["gva"], "gva_steps", H=2, HV=4)
    N, P, T = 6, 8, 4
    x = oracle.add_gates(make_inputs(scaled(w, "gva_steps", B=N, T=T, init="none"), seed=3))
    gen = torch.Generator().manual_seed(4)
    pool = torch.randn(P, w.HV, w.K, w.V, generator=gen) * 0.05
    idx = torch.tensor([5, 1, -1, 0, 7, 3], dtype=torch.int32)
    pool_d = pool.to(DEV).contiguous()
    outs = []
    for t in range(T):
        o = gdn.fused_recurrent_gated_delta_rule_update(
            x["q"][:, t].to(DEV), x["k"][:, t].to(DEV), x["v"][:, t].to(DEV), x["g"][:, t].to(DEV),
            x["beta"][:, t].to(DEV), pool_d, idx.to(DEV), scale=x["scale"],
            use_qk_l2norm_in_kernel=x["use_l2norm"])
        outs.append(o.float().cpu())
    torch.cuda.synchronize()
    valid = [0, 1, 3, 4, 5]
    sel = torch.tensor(valid)
    o_ref, f_ref = oracle.recurrent(x["q"][sel], x["k"][sel], x["v"][sel], x["g"][sel], x["beta"][sel],
                                    scale=x["scale"], use_l2norm=x["use_l2norm"],
                                    initial_state=pool[idx[sel].long()].double())
    o_gpu = torch.stack(outs, 1)[sel].numpy().astype(np.float64)
    eo = float(np.abs(o_gpu - o_ref).max())
    ef = float(np.abs(pool_d.cpu()[idx[sel].long()].numpy().astype(np.float64) - f_ref).max())
    _say(f"    4 steps: max|do|={eo:.3e}  max|dS|={ef:.3e}")
    assert eo <= 2e-2 and ef <= 1e-2
    assert torch.all(torch.stack(outs, 1)[2] == 0)


def test_decode_continues_prefill():
    """Prefill of T-1 tokens, its final state placed in the pool, then one
    decode step: the last output row and the state match a T-token prefill."""
    gdn = _gdn()
    w = scaled(WORKLOADS["gva"], "gva_cont", H=2, HV=4)
    B, T = 3, 130
    x = oracle.add_gates(make_inputs(scaled(w, "gva_cont", B=B, T=T), seed=5))
    d = lambda t: t.to(DEV)
    o_full, f_full = gdn.chunk_gated_delta_rule(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), d(x["beta"]),
                                                scale=x["scale"], initial_state=d(x["initial_state"]),
                                                use_qk_l2norm_in_kernel=True)
    _, f_pre = gdn.chunk_gated_delta_rule(d(x["q"][:, :-1]), d(x["k"][:, :-1]), d(x["v"][:, :-1]),
                                          d(x["g"][:, :-1]), d(x["beta"][:, :-1]), scale=x["scale"],
                                          initial_state=d(x["initial_state"]), use_qk_l2norm_in_kernel=True)
    pool = torch.zeros(5, w.HV, w.K, w.V, device=DEV)
    idx = torch.tensor([4, 0, 2], dtype=torch.int32, device=DEV)
    pool[idx.long()] = f_pre
    o_last = gdn.fused_recurrent_gated_delta_rule_update(
        d(x["q"][:, -1]), d(x["k"][:, -1]), d(x["v"][:, -1]), d(x["g"][:, -1]), d(x["beta"][:, -1]),
        pool, idx, scale=x["scale"], use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    eo = float((o_last.float() - o_full[:, -1].float()).abs().max())
    ef = float((pool[idx.long()] - f_full).abs().max())
    _say(f"    prefill+decode vs prefill: max|do|={eo:.3e}  max|dS|={ef:.3e}")
    assert eo <= 2e-2 and ef <= 1e-2


def test_decode_empty_batch():
    gdn = _gdn()
    e = torch.empty(0, 2, 64, dtype=torch.bfloat16, device=DEV)
    v = torch.empty(0, 4, 64, dtype=torch.bfloat16, device=DEV)
    g = torch.empty(0, 4, device=DEV)
    pool = torch.zeros(2, 4, 64, 64, device=DEV)
    o = gdn.fused_recurrent_gated_delta_rule_update(e, e, v, g, g, pool, torch.empty(0, dtype=torch.int32,
                                                                                      device=DEV))
    torch.cuda.synchronize()
    assert o.shape == (0, 4, 64) and torch.count_nonzero(pool) == 0


@pytest.mark.parametrize("name", ["decode", "decode_bf16pool"])
def test_decode_bench_workloads_full_size(name):
    """The decode steps the benchmark times, at their size (256 rows, 8 of them
    padding, a 512-slot fp32 or bf16 pool, 32 value heads), from the same input
    generator; the gates come from the oracle and feed both sides."""
    from workloads import DECODE_WORKLOADS, make_decode_inputs
    gdn = _gdn()
    w = DECODE_WORKLOADS[name]
    x = make_decode_inputs(w, seed=0, device=DEV)
    g, beta = oracle.gating(x["A_log"].cpu(), x["dt_bias"].cpu(), x["a"].float().cpu(), x["b"].float().cpu())
    g = torch.as_tensor(g, dtype=torch.float32)
    beta = torch.as_tensor(beta, dtype=torch.float32)
    pool0 = x["pool"].cpu()
    idx = x["idx"].cpu()
    _say(f"[decode-full] {name}: N={w.N} pool={w.pool_size} ({pool0.dtype})")
    pool = x["pool"]
    o = gdn.fused_recurrent_gated_delta_rule_update(x["q"], x["k"], x["v"], g.to(DEV), beta.to(DEV), pool, x["idx"],
                                                    scale=x["scale"], use_qk_l2norm_in_kernel=x["use_l2norm"])
    torch.cuda.synchronize()
    o, pool_after = o.float().cpu(), pool.float().cpu()
    cpu = lambda t: t.float().cpu().unsqueeze(1)
    o_ref, after_ref = oracle.recurrent_pool(cpu(x["q"]), cpu(x["k"]), cpu(x["v"]), g.unsqueeze(1),
                                             beta.unsqueeze(1), pool0, idx, scale=x["scale"],
                                             use_l2norm=x["use_l2norm"])
    valid = [r for r in range(w.N) if 0 <= int(idx[r]) < w.pool_size]
    assert len(valid) == w.N - w.n_pad
    to, tf = TOL[torch.bfloat16]
    eo = float(np.abs(o[valid].numpy().astype(np.float64) - o_ref[valid, 0]).max())
    slots = idx[valid].long()
    ef = float(np.abs(pool_after[slots].numpy().astype(np.float64) - after_ref[slots.numpy()]).max())
    _say(f"    max|do|={eo:.3e} (bar {to})  max|dS|={ef:.3e} (bar {tf})")
    assert eo <= to and ef <= tf
    pads = [r for r in range(w.N) if r not in valid]
    assert torch.all(o[pads] == 0)
    untouched = torch.ones(w.pool_size, dtype=torch.bool)
    untouched[slots] = False
    assert torch.equal(pool_after[untouched], pool0[untouched].float())
