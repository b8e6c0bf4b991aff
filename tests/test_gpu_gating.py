"""GPU parity of the gate computation (g = -exp(A_log) softplus(a + dt_bias),
beta = sigmoid(b)): the stand-alone gating kernel against the oracle's float64
gates, and the prefill and decode kernels with in-kernel gating against the
oracle's gated recurrence, through the C ABI.

Bars: the gating kernel computes in fp32, so g within 4e-6 relative (+1e-7
absolute) and beta within 1e-6 of the float64 values; the gated prefill and
decode keep the bars of the un-gated paths (bf16 2e-2 on o, 1e-2 on the
state; fp32 check mode 1e-4 on both).
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


def _raw(x):
    return dict(A_log=x["A_log"].to(DEV), dt_bias=x["dt_bias"].to(DEV))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_gating_kernel_matches_oracle(dtype):
    gdn = _gdn()
    gen = torch.Generator().manual_seed(11)
    rows, HV = 4099, 6                        # rows * HV not a multiple of the 4 elements a thread takes
    a = torch.randn(rows, HV, generator=gen) * 3
    b = torch.randn(rows, HV, generator=gen) * 3
    # tails and exact points: large |a + dt_bias| and |b|, zeros
    a[:4] = torch.tensor([[100.0], [-100.0], [0.0], [30.0]])
    b[:4] = torch.tensor([[100.0], [-100.0], [0.0], [-30.0]])
    a, b = a.to(torch.bfloat16).to(dtype), b.to(torch.bfloat16).to(dtype)
    A_log = torch.rand(HV, generator=gen) * float(np.log(16.0))
    dt_bias = torch.rand(HV, generator=gen)
    g, beta = gdn.fused_gdn_gating(A_log.to(DEV), a.to(DEV), b.to(DEV), dt_bias.to(DEV))
    torch.cuda.synchronize()
    g_ref, b_ref = oracle.gating(A_log, dt_bias, a, b)
    eg = np.abs(g.cpu().numpy().astype(np.float64) - g_ref)
    eb = float(np.abs(beta.cpu().numpy().astype(np.float64) - b_ref).max())
    rel = float((eg / (np.abs(g_ref) + 1e-30)).max())
    _say(f"    gating {dtype}: max rel|dg|={rel:.2e}  max|dbeta|={eb:.2e}")
    assert np.all(eg <= 4e-6 * np.abs(g_ref) + 1e-7) and eb <= 1e-6
    # a [..., HV] of more than two dimensions and a single row
    g3, b3 = gdn.fused_gdn_gating(A_log.to(DEV), a[:6].reshape(2, 3, HV).to(DEV), b[:6].reshape(2, 3, HV).to(DEV),
                                  dt_bias.to(DEV))
    assert g3.shape == (2, 3, HV) and torch.equal(g3.reshape(6, HV), g[:6])


def _prefill(x, dtype, fused=True):
    gdn = _gdn()
    d = lambda t: None if t is None else t.to(DEV)
    kw = dict(scale=x["scale"], initial_state=d(x["initial_state"]), cu_seqlens=d(x["cu_seqlens"]),
              use_qk_l2norm_in_kernel=x["use_l2norm"])
    q, k, v = (x[n].to(DEV, dtype) for n in ("q", "k", "v"))
    a, b = x["a"].to(DEV, dtype), x["b"].to(DEV, dtype)
    if fused:
        o, fin = gdn.chunk_gated_delta_rule(q, k, v, A_log=x["A_log"].to(DEV), dt_bias=x["dt_bias"].to(DEV),
                                            a_raw=a, b_raw=b, **kw)
    else:
        g, beta = gdn.fused_gdn_gating(x["A_log"].to(DEV), a, b, x["dt_bias"].to(DEV))
        o, fin = gdn.chunk_gated_delta_rule(q, k, v, g, beta, **kw)
    torch.cuda.synchronize()
    return o, fin


SMALL = {
    "tiny": (WORKLOADS["tiny"], (torch.bfloat16, torch.float32)),
    "gva_ragged": (scaled(WORKLOADS["gva"], "gva_ragged", B=2, T=300, H=2, HV=4), (torch.bfloat16, torch.float32)),
    "varlen_mix": (scaled(WORKLOADS["varlen"], "varlen_mix", H=2, HV=4, lengths=(1, 64, 65, 127, 0, 200, 3, 129)),
                   (torch.bfloat16, torch.float32)),
    "wide_sat": (scaled(WORKLOADS["wide_stable"], "wide_sat", B=2, T=140, H=2, HV=4), (torch.bfloat16,)),
    "odd_hv_fp32": (scaled(WORKLOADS["gva"], "odd_hv", B=2, T=130, H=1, HV=3, K=128, V=64), (torch.float32,)),
}
CASES = [(n, d) for n, (_, ds) in SMALL.items() for d in ds]


@pytest.mark.parametrize("name,dtype", CASES, ids=[f"{n}-{'bf16' if d == torch.bfloat16 else 'fp32'}"
                                                    for n, d in CASES])
def test_prefill_gated_parity(name, dtype):
    w = SMALL[name][0]
    x = make_inputs(w, seed=7, io_dtype=torch.float32)
    _say(f"[gated prefill] {name} dtype={dtype} lens={x['lens'][:8]}")
    o, fin = _prefill(x, dtype)
    o_ref, f_ref = oracle.recurrent_gated(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"], x["b"],
                                          scale=x["scale"], use_l2norm=x["use_l2norm"],
                                          initial_state=x["initial_state"],
                                          cu_seqlens=None if x["cu_seqlens"] is None else x["cu_seqlens"].numpy())
    eo = float(np.abs(o.float().cpu().numpy().astype(np.float64) - o_ref).max())
    ef = float(np.abs(fin.cpu().numpy().astype(np.float64) - f_ref).max())
    to, tf = TOL[dtype]
    _say(f"    max|do|={eo:.3e} (bar {to})  max|dS|={ef:.3e} (bar {tf})")
    assert eo <= to and ef <= tf


def test_prefill_gated_equals_separate_gating():
    """In-kernel gates and the gating kernel's gates drive the chunk kernel
    to the same result (the same fp32 gate arithmetic; only rounding order
    can differ)."""
    w = scaled(WORKLOADS["gva"], "gva_sep", B=2, T=333, H=2, HV=4)
    x = make_inputs(w, seed=8)
    o1, f1 = _prefill(x, torch.bfloat16, fused=True)
    o2, f2 = _prefill(x, torch.bfloat16, fused=False)
    do = float((o1.float() - o2.float()).abs().max())
    df = float((f1 - f2).abs().max())
    _say(f"    fused vs separate gating: max|do|={do:.3e} max|dS|={df:.3e}")
    assert do <= 4e-3 and df <= 1e-4


def test_prefill_gated_full_size_sampled():
    """The GVA workload at full size with in-kernel gating, as the benchmark
    launches it; sampled (sequence, value head) units against the oracle."""
    gdn = _gdn()
    w = WORKLOADS["gva"]
    _say("[gated prefill full] gva: generating on the GPU")
    x = make_inputs(w, seed=0, device="cuda:0")
    o, fin = gdn.chunk_gated_delta_rule(x["q"], x["k"], x["v"], A_log=x["A_log"], dt_bias=x["dt_bias"],
                                        a_raw=x["a"], b_raw=x["b"], scale=x["scale"],
                                        initial_state=x["initial_state"], use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(fin).all()
    HV, G = w.HV, w.HV // w.H
    worst_o = worst_f = 0.0
    for u in (0, 37, 64 + 31, 4 * HV - 1):
        n, j = divmod(u, HV)
        jk = j // G
        sl = lambda t, h: t[n:n + 1, :, h:h + 1].cpu()
        o_ref, f_ref = oracle.recurrent_gated(sl(x["q"], jk), sl(x["k"], jk), sl(x["v"], j),
                                              x["A_log"][j:j + 1].cpu(), x["dt_bias"][j:j + 1].cpu(),
                                              sl(x["a"], j), sl(x["b"], j), scale=x["scale"], use_l2norm=True,
                                              initial_state=x["initial_state"][n:n + 1, j:j + 1].cpu(),
                                              nthreads=8)
        eo = float(np.abs(o[n, :, j].float().cpu().numpy() - o_ref[0, :, 0]).max())
        ef = float(np.abs(fin[n, j].cpu().numpy() - f_ref[0, 0]).max())
        worst_o, worst_f = max(worst_o, eo), max(worst_f, ef)
        _say(f"    unit n={n} j={j}: max|do|={eo:.3e} max|dS|={ef:.3e}")
    assert worst_o <= 2e-2 and worst_f <= 1e-2


def _decode_case(seed=9):
    w = scaled(WORKLOADS["gva"], "gva_dec_gated", B=40, T=1, H=4, HV=8, init="none")
    x = make_inputs(w, seed=seed, io_dtype=torch.float32)
    gen = torch.Generator().manual_seed(seed + 1)
    pool = torch.randn(48, w.HV, w.K, w.V, generator=gen) * 0.05
    idx = torch.randperm(48, generator=gen)[:40].to(torch.int32)
    idx[3] = -1
    idx[20] = 48 + 5
    return x, pool, idx


def _decode(x, pool, idx, dtype, fused=True):
    gdn = _gdn()
    pool_d = pool.to(DEV).contiguous()
    q, k, v = (x[n][:, 0].to(DEV, dtype) for n in ("q", "k", "v"))
    a, b = x["a"][:, 0].to(DEV, dtype), x["b"][:, 0].to(DEV, dtype)
    kw = dict(scale=x["scale"], use_qk_l2norm_in_kernel=x["use_l2norm"])
    if fused:
        o = gdn.fused_recurrent_gated_delta_rule_update(q, k, v, None, None, pool_d, idx.to(DEV),
                                                        A_log=x["A_log"].to(DEV), dt_bias=x["dt_bias"].to(DEV),
                                                        a_raw=a, b_raw=b, **kw)
    else:
        g, beta = gdn.fused_gdn_gating(x["A_log"].to(DEV), a, b, x["dt_bias"].to(DEV))
        o = gdn.fused_recurrent_gated_delta_rule_update(q, k, v, g, beta, pool_d, idx.to(DEV), **kw)
    torch.cuda.synchronize()
    return o.float().cpu(), pool_d.cpu()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_decode_gated_parity(dtype):
    x, pool, idx = _decode_case()
    o, pool_after = _decode(x, pool, idx, dtype)
    valid = [r for r in range(idx.numel()) if 0 <= int(idx[r]) < pool.shape[0]]
    sel = torch.tensor(valid)
    o_ref, f_ref = oracle.recurrent_gated(x["q"][sel], x["k"][sel], x["v"][sel], x["A_log"], x["dt_bias"],
                                          x["a"][sel], x["b"][sel], scale=x["scale"], use_l2norm=x["use_l2norm"],
                                          initial_state=pool[idx[sel].long()].double())
    eo = float(np.abs(o[valid].numpy().astype(np.float64) - o_ref[:, 0]).max())
    ef = float(np.abs(pool_after[idx[sel].long()].numpy().astype(np.float64) - f_ref).max())
    to, tf = TOL[dtype]
    _say(f"    gated decode {dtype}: max|do|={eo:.3e} (bar {to})  max|dS|={ef:.3e} (bar {tf})")
    assert eo <= to and ef <= tf
    assert torch.all(o[[3, 20]] == 0)
    untouched = torch.ones(pool.shape[0], dtype=torch.bool)
    untouched[idx[sel].long()] = False
    assert torch.equal(pool_after[untouched], pool[untouched])


def test_decode_gated_equals_separate_gating():
    x, pool, idx = _decode_case(seed=12)
    o1, p1 = _decode(x, pool, idx, torch.bfloat16, fused=True)
    o2, p2 = _decode(x, pool, idx, torch.bfloat16, fused=False)
    do, dp = float((o1 - o2).abs().max()), float((p1 - p2).abs().max())
    _say(f"    decode fused vs separate gating: max|do|={do:.3e} max|dS|={dp:.3e}")
    assert do <= 4e-3 and dp <= 1e-5
