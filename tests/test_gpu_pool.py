"""GPU parity of the state-pool entry points (prefill and decode reading and
updating slot-indexed states in place, fp32 or bf16 pools) against the
oracle's pool form, through the C ABI.

Bars: as prefill/decode (bf16 inputs 2e-2 on o, 1e-2 on the state; fp32 check
mode 1e-4).  A bf16 pool stores each final state rounded to bf16, so its state
bar adds one bf16 rounding: 1e-2 + 2^-8 |S| (and the fp32-mode bar becomes
1e-4 + 2^-8 |S|).  Slots that no valid sequence names must stay bit-identical.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = {torch.bfloat16: (2e-2, 1e-2), torch.float32: (1e-4, 1e-4)}


def _gdn():
    import gated_deltanet_chunked_delta_amd as gdn
    gdn.load_library()
    return gdn


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _pool(P, w, pool_dtype, seed):
    gen = torch.Generator().manual_seed(seed)
    return (torch.randn(P, w.HV, w.K, w.V, generator=gen) * 0.05).to(pool_dtype)


def _check_pool(after, ref, pool0, idx, io_dtype, pool_dtype, tag):
    P = pool0.shape[0]
    valid = [int(s) for s in idx.tolist() if 0 <= s < P]
    got = after.float().numpy().astype(np.float64)
    tf = TOL[io_dtype][1]
    err = np.abs(got[valid] - ref[valid])
    bar = tf + (2.0 ** -8 * np.abs(ref[valid]) if pool_dtype == torch.bfloat16 else 0.0)
    ratio = float((err / bar).max()) if len(valid) else 0.0
    _say(f"    {tag}: max|dS|={float(err.max()) if len(valid) else 0:.3e} (worst err/bar {ratio:.2f})")
    assert np.all(err <= bar)
    untouched = [s for s in range(P) if s not in valid]
    assert torch.equal(after[untouched], pool0[untouched])


PREFILL = {
    "varlen": scaled(WORKLOADS["varlen"], "varlen_pool", H=2, HV=4, lengths=(1, 64, 65, 127, 0, 200, 3, 129)),
    "gva": scaled(WORKLOADS["gva"], "gva_pool", B=3, T=150, H=2, HV=4, init="none"),
}
CASES = [(n, io, pd, ri) for n in PREFILL for io in (torch.bfloat16, torch.float32)
         for pd in (torch.float32, torch.bfloat16) for ri in (True, False)]


def _id(c):
    n, io, pd, ri = c
    return f"{n}-io_{str(io)[6:]}-pool_{str(pd)[6:]}-{'read' if ri else 'zero'}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_prefill_pool_parity(case):
    name, io, pd, read_initial = case
    gdn = _gdn()
    w = PREFILL[name]
    x = oracle.add_gates(make_inputs(w, seed=21, io_dtype=torch.float32))
    N = x["N"]
    P = N + 5
    pool0 = _pool(P, w, pd, seed=22)
    idx = torch.randperm(P, generator=torch.Generator().manual_seed(23))[:N].to(torch.int32)
    idx[1] = -1                       # a sequence with no state slot
    if N > 3:
        idx[3] = P + 2                # a slot past the pool: also none
    _say(f"[pool prefill] {_id(case)} N={N} P={P} idx={idx.tolist()}")
    pool_d = pool0.to(DEV).contiguous()
    d = lambda t: None if t is None else t.to(DEV)
    o, none = gdn.chunk_gated_delta_rule(x["q"].to(DEV, io), x["k"].to(DEV, io), x["v"].to(DEV, io),
                                         d(x["g"]), d(x["beta"]), scale=x["scale"], cu_seqlens=d(x["cu_seqlens"]),
                                         use_qk_l2norm_in_kernel=x["use_l2norm"], ssm_state_pool=pool_d,
                                         ssm_state_indices=idx.to(DEV), read_initial_state=read_initial)
    torch.cuda.synchronize()
    assert none is None
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].numpy()
    o_ref, after_ref = oracle.recurrent_pool(x["q"], x["k"], x["v"], x["g"], x["beta"], pool0, idx,
                                             read_initial=read_initial, scale=x["scale"],
                                             use_l2norm=x["use_l2norm"], cu_seqlens=cu)
    eo = float(np.abs(o.float().cpu().numpy().astype(np.float64) - o_ref).max())
    _say(f"    max|do|={eo:.3e} (bar {TOL[io][0]})")
    assert eo <= TOL[io][0]
    _check_pool(pool_d.cpu(), after_ref, pool0, idx, io, pd, "pool")


def test_prefill_pool_gated_bf16_serving_call():
    """The serving combination: packed sequences, gates computed in the
    kernel from the raw inputs, a bf16 pool read and updated in place."""
    gdn = _gdn()
    w = PREFILL["varlen"]
    x = make_inputs(w, seed=24)
    N = x["N"]
    pool0 = _pool(N + 2, w, torch.bfloat16, seed=25)
    idx = torch.arange(N, dtype=torch.int32).flip(0)
    pool_d = pool0.to(DEV).contiguous()
    d = lambda t: t.to(DEV)
    o, _ = gdn.chunk_gated_delta_rule(d(x["q"]), d(x["k"]), d(x["v"]), A_log=d(x["A_log"]), dt_bias=d(x["dt_bias"]),
                                      a_raw=d(x["a"]), b_raw=d(x["b"]), scale=x["scale"],
                                      cu_seqlens=d(x["cu_seqlens"]), use_qk_l2norm_in_kernel=True,
                                      ssm_state_pool=pool_d, ssm_state_indices=idx.to(DEV))
    torch.cuda.synchronize()
    g, beta = oracle.gating(x["A_log"], x["dt_bias"], x["a"], x["b"])
    o_ref, after_ref = oracle.recurrent_pool(x["q"], x["k"], x["v"], g.astype(np.float32), beta.astype(np.float32),
                                             pool0, idx, scale=x["scale"], use_l2norm=True,
                                             cu_seqlens=x["cu_seqlens"].numpy())
    eo = float(np.abs(o.float().cpu().numpy().astype(np.float64) - o_ref).max())
    _say(f"    gated bf16-pool prefill: max|do|={eo:.3e}")
    assert eo <= 2e-2
    _check_pool(pool_d.cpu(), after_ref, pool0, idx, torch.bfloat16, torch.bfloat16, "pool")


@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32], ids=["io_bf16", "io_fp32"])
def test_decode_bf16_pool_parity(io):
    gdn = _gdn()
    w = scaled(WORKLOADS["gva"], "gva_dec_pool", B=40, T=1, H=4, HV=8, init="none")
    x = oracle.add_gates(make_inputs(w, seed=26, io_dtype=torch.float32))
    pool0 = _pool(48, w, torch.bfloat16, seed=27)
    idx = torch.randperm(48, generator=torch.Generator().manual_seed(28))[:40].to(torch.int32)
    idx[5], idx[17] = -1, 48 + 1
    pool_d = pool0.to(DEV).contiguous()
    o = gdn.fused_recurrent_gated_delta_rule_update(
        x["q"][:, 0].to(DEV, io), x["k"][:, 0].to(DEV, io), x["v"][:, 0].to(DEV, io), x["g"][:, 0].to(DEV),
        x["beta"][:, 0].to(DEV), pool_d, idx.to(DEV), scale=x["scale"], use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    o_ref, after_ref = oracle.recurrent_pool(x["q"], x["k"], x["v"], x["g"], x["beta"], pool0, idx,
                                             scale=x["scale"], use_l2norm=True)
    valid = [r for r in range(40) if 0 <= int(idx[r]) < 48]
    eo = float(np.abs(o.float().cpu().numpy()[valid] - o_ref[valid, 0]).max())
    _say(f"    bf16-pool decode ({io}): max|do|={eo:.3e}")
    assert eo <= TOL[io][0]
    assert torch.all(o.cpu()[[5, 17]] == 0)
    _check_pool(pool_d.cpu(), after_ref, pool0, idx, io, torch.bfloat16, "pool")


def test_prefill_then_decode_on_a_bf16_pool():
    """Prefill T-1 tokens into a bf16 pool (read_initial off: a new request),
    then one gated decode step from the pool: the oracle rounds the state to
    bf16 between the two, as the pool stores it."""
    gdn = _gdn()
    w = scaled(WORKLOADS["gva"], "gva_pd", B=3, T=97, H=2, HV=4, init="none")
    x = make_inputs(w, seed=29)
    P = 6
    pool_d = torch.full((P, w.HV, w.K, w.V), 7.0, dtype=torch.bfloat16, device=DEV)
    idx = torch.tensor([4, 0, 2], dtype=torch.int32)
    d = lambda t: t.to(DEV)
    gk = dict(A_log=d(x["A_log"]), dt_bias=d(x["dt_bias"]))
    gdn.chunk_gated_delta_rule(d(x["q"][:, :-1]), d(x["k"][:, :-1]), d(x["v"][:, :-1]), a_raw=d(x["a"][:, :-1]),
                               b_raw=d(x["b"][:, :-1]), scale=x["scale"], use_qk_l2norm_in_kernel=True,
                               ssm_state_pool=pool_d, ssm_state_indices=d(idx), read_initial_state=False, **gk)
    o_last = gdn.fused_recurrent_gated_delta_rule_update(
        d(x["q"][:, -1]), d(x["k"][:, -1]), d(x["v"][:, -1]), None, None, pool_d, d(idx), scale=x["scale"],
        use_qk_l2norm_in_kernel=True, a_raw=d(x["a"][:, -1]), b_raw=d(x["b"][:, -1]), **gk)
    torch.cuda.synchronize()
    g, beta = oracle.gating(x["A_log"], x["dt_bias"], x["a"], x["b"])
    g, beta = torch.from_numpy(g.astype(np.float32)), torch.from_numpy(beta.astype(np.float32))
    _, f_pre = oracle.recurrent(x["q"][:, :-1], x["k"][:, :-1], x["v"][:, :-1], g[:, :-1], beta[:, :-1],
                                scale=x["scale"], use_l2norm=True)
    s_mid = torch.from_numpy(f_pre).to(torch.bfloat16).float().numpy()        # the pool's bf16 copy
    o_ref, f_ref = oracle.recurrent(x["q"][:, -1:], x["k"][:, -1:], x["v"][:, -1:], g[:, -1:], beta[:, -1:],
                                    scale=x["scale"], use_l2norm=True, initial_state=s_mid)
    eo = float(np.abs(o_last.float().cpu().numpy() - o_ref[:, 0]).max())
    got = pool_d[idx.long().to(DEV)].float().cpu().numpy()
    ef = np.abs(got - f_ref)
    _say(f"    prefill+decode on bf16 pool: max|do|={eo:.3e} max|dS|={float(ef.max()):.3e}")
    assert eo <= 2e-2 and np.all(ef <= 1e-2 + 2.0 ** -8 * np.abs(f_ref))
    assert torch.all(pool_d[[1, 3, 5]].float() == 7.0)


def test_prefill_pool_gated_bf16_full_size_sampled():
    """The serving call at the size of the packed workload (64 sequences,
    62,386 tokens, 32 value heads): gates computed in the kernel, a bf16 pool
    of 80 slots read and updated in place through a shuffled slot map; sampled
    (sequence, value head) units against the oracle, every slot no sequence
    names bit-identical."""
    gdn = _gdn()
    w = WORKLOADS["varlen"]
    x = make_inputs(w, seed=0, device="cuda:0")
    N, HV = x["N"], w.HV
    P = N + 16
    pool0 = _pool(P, w, torch.bfloat16, seed=26)
    idx = torch.randperm(P, generator=torch.Generator().manual_seed(27))[:N].to(torch.int32)
    pool_d = pool0.to(DEV).contiguous()
    _say(f"[pool-full] varlen: N={N} tokens={sum(x['lens'])} pool={P} bf16")
    o, _ = gdn.chunk_gated_delta_rule(x["q"], x["k"], x["v"], A_log=x["A_log"], dt_bias=x["dt_bias"],
                                      a_raw=x["a"], b_raw=x["b"], scale=x["scale"], cu_seqlens=x["cu_seqlens"],
                                      use_qk_l2norm_in_kernel=True, ssm_state_pool=pool_d,
                                      ssm_state_indices=idx.to(DEV))
    torch.cuda.synchronize()
    after = pool_d.cpu()
    starts = [int(c) for c in x["cu_seqlens"].tolist()]
    longest = int(np.argmax(x["lens"]))
    G = HV // w.H
    for n, j in ((0, 0), (longest, HV // 2), (N - 1, HV - 1)):
        t0, t1 = starts[n], starts[n + 1]
        jk = j // G
        rows = lambda t, h: t[0, t0:t1, h:h + 1].unsqueeze(0).float().cpu()
        g, beta = oracle.gating(x["A_log"][j:j + 1].cpu(), x["dt_bias"][j:j + 1].cpu(), rows(x["a"], j),
                                rows(x["b"], j))   # [1, L, 1]
        s0 = pool0[int(idx[n]), j:j + 1].unsqueeze(0).float()
        o_ref, f_ref = oracle.recurrent(rows(x["q"], jk), rows(x["k"], jk), rows(x["v"], j),
                                        torch.as_tensor(g, dtype=torch.float32),
                                        torch.as_tensor(beta, dtype=torch.float32), scale=x["scale"],
                                        use_l2norm=True, initial_state=s0)
        og = o[0, t0:t1, j].float().cpu().numpy().astype(np.float64)
        eo = float(np.abs(og - o_ref[0, :, 0]).max()) if t1 > t0 else 0.0
        ref = f_ref[0, 0]
        err = np.abs(after[int(idx[n]), j].float().numpy().astype(np.float64) - ref)
        ratio = float((err / (1e-2 + 2.0 ** -8 * np.abs(ref))).max())
        _say(f"    unit n={n} j={j} len={t1 - t0}: max|do|={eo:.3e}  state err/bar {ratio:.2f}")
        assert eo <= 2e-2 and ratio <= 1.0
    untouched = [s for s in range(P) if s not in set(idx.tolist())]
    assert torch.equal(after[untouched], pool0[untouched])
