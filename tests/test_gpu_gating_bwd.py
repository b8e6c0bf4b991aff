"""GPU parity of the gate-input gradients (gdn_gating_bwd through the C ABI)
against the oracle's float64 chain rule (oracle.gating_bwd, pinned to finite
differences of the gate function).

Bars: the kernels compute in fp32 and round da, db once to the inputs' dtype,
so da, db within 2^-8 + 1e-5 of max|ref| in bf16 and 1e-5 in fp32; the per-head
sums dA_log and ddt_bias are fp32 sums over the rows, within 1e-5 of the sum of
the absolute values of their terms.
"""
import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _gdn():
    import gated_deltanet_chunked_delta_amd as gdn
    gdn.load_library()
    return gdn


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(rows, HV, dtype, seed):
    gen = torch.Generator().manual_seed(seed)
    A_log = torch.rand(HV, generator=gen) * float(np.log(16.0))
    dt_bias = torch.rand(HV, generator=gen)
    a = torch.randn(rows, HV, generator=gen).to(dtype)
    b = (torch.randn(rows, HV, generator=gen) * 2).to(dtype)
    dg = torch.randn(rows, HV, generator=gen)
    dbeta = torch.randn(rows, HV, generator=gen)
    return A_log, dt_bias, a, b, dg, dbeta


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("rows,HV", [(231, 3), (4099, 32), (130, 300), (1, 5)],
                         ids=["ragged_odd_heads", "gva_heads", "wide_heads", "one_row"])
def test_gating_bwd_matches_oracle(rows, HV, dtype):
    gdn = _gdn()
    A_log, dt_bias, a, b, dg, dbeta = _inputs(rows, HV, dtype, seed=rows + HV)
    _say(f"[gating-bwd] rows={rows} HV={HV} dtype={dtype}")
    da, db, dA, ddt = gdn.fused_gdn_gating_bwd(A_log.to(DEV), a.to(DEV), b.to(DEV), dt_bias.to(DEV),
                                               dg.to(DEV), dbeta.to(DEV))
    torch.cuda.synchronize()
    assert da.dtype == dtype and db.dtype == dtype and tuple(da.shape) == (rows, HV)
    rda, rdb, rdA, rddt = oracle.gating_bwd(A_log, dt_bias, a.float(), b.float(), dg, dbeta)
    bar = 2.0 ** -8 + 1e-5 if dtype == torch.bfloat16 else 1e-5
    for name, got, ref in (("da", da, rda), ("db", db, rdb)):
        err = float(np.abs(got.float().cpu().numpy() - ref).max()) / max(float(np.abs(ref).max()), 1e-30)
        _say(f"    {name}: rel max err {err:.2e} (bar {bar:.1e})")
        assert err <= bar, name
    g, _ = oracle.gating(A_log, dt_bias, a.float(), b.float())
    scales = {"dA_log": np.abs(dg.double().numpy() * g).sum(axis=0), "ddt_bias": np.abs(rda).sum(axis=0)}
    for name, got, ref in (("dA_log", dA, rdA), ("ddt_bias", ddt, rddt)):
        d = np.abs(got.cpu().numpy() - ref)
        _say(f"    {name}: max |d| / sum|terms| {float((d / scales[name]).max()):.2e}")
        assert np.all(d <= 1e-5 * scales[name] + 1e-30), name


def test_gating_bwd_no_rows_gives_zero_sums():
    gdn = _gdn()
    A_log, dt_bias, a, b, dg, dbeta = _inputs(0, 4, torch.bfloat16, seed=3)
    da, db, dA, ddt = gdn.fused_gdn_gating_bwd(A_log.to(DEV), a.to(DEV), b.to(DEV), dt_bias.to(DEV),
                                               dg.to(DEV), dbeta.to(DEV))
    torch.cuda.synchronize()
    assert da.numel() == 0 and torch.equal(dA.cpu(), torch.zeros(4)) and torch.equal(ddt.cpu(), torch.zeros(4))


def test_gating_bwd_deterministic_and_matches_chunk_bwd_gate_shapes():
    """Two calls agree bit for bit; fed with the dg, dbeta of the chunked
    backward pass ([B, T, HV]) it returns a, b's shapes."""
    gdn = _gdn()
    A_log, dt_bias, a, b, dg, dbeta = _inputs(2 * 700, 8, torch.bfloat16, seed=9)
    args = [A_log.to(DEV), a.reshape(2, 700, 8).to(DEV), b.reshape(2, 700, 8).to(DEV), dt_bias.to(DEV),
            dg.reshape(2, 700, 8).to(DEV), dbeta.reshape(2, 700, 8).to(DEV)]
    r1 = gdn.fused_gdn_gating_bwd(*args)
    r2 = gdn.fused_gdn_gating_bwd(*args)
    torch.cuda.synchronize()
    assert tuple(r1[0].shape) == (2, 700, 8) and tuple(r1[1].shape) == (2, 700, 8)
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)


def test_training_chain_gates_to_gate_inputs():
    """GPU gating, the chunked backward pass and the gate-input gradients in a
    row (fp32 I/O), against the oracle's float64 chain: gates, backward,
    gate-input gradients.  The chunked backward's bar (1e-4 of max|dg|, max|dbeta|
    per element) carries through the linear maps that follow it."""
    from oracle.backward import backward as oracle_backward
    from workloads import WORKLOADS, make_grad_inputs, make_inputs, scaled

    gdn = _gdn()
    w = scaled(WORKLOADS["gva"], "chain", B=2, T=150, H=2, HV=4)
    x = make_grad_inputs(make_inputs(w, seed=5, io_dtype=torch.float32), seed=105)
    dev = lambda t: None if t is None else t.to(DEV)
    g, beta = gdn.fused_gdn_gating(dev(x["A_log"]), dev(x["a"]), dev(x["b"]), dev(x["dt_bias"]))
    out = gdn.chunk_gated_delta_rule_bwd(dev(x["q"]), dev(x["k"]), dev(x["v"]), g, beta, dev(x["do"]),
                                         dht=dev(x["dht"]), scale=x["scale"], initial_state=dev(x["initial_state"]),
                                         use_qk_l2norm_in_kernel=x["use_l2norm"])
    dg, dbeta = out[3], out[4]
    da, db, dA, ddt = gdn.fused_gdn_gating_bwd(dev(x["A_log"]), dev(x["a"]), dev(x["b"]), dev(x["dt_bias"]),
                                               dg, dbeta)
    torch.cuda.synchronize()

    g64, b64 = oracle.gating(x["A_log"], x["dt_bias"], x["a"], x["b"])
    ref = oracle_backward(x["q"], x["k"], x["v"], torch.from_numpy(g64), torch.from_numpy(b64), x["do"],
                          dht=x["dht"], scale=x["scale"], use_l2norm=x["use_l2norm"],
                          initial_state=x["initial_state"])
    rda, rdb, rdA, rddt = oracle.gating_bwd(x["A_log"], x["dt_bias"], x["a"], x["b"], ref["dg"], ref["dbeta"])
    mdg, mdb = float(np.abs(ref["dg"]).max()), float(np.abs(ref["dbeta"]).max())
    A = np.exp(x["A_log"].double().numpy())
    fac = A * oracle.sigmoid(x["a"].double().numpy() + x["dt_bias"].double().numpy())   # |d g / d a|
    bb = b64 * (1 - b64)                                                                  # d beta / d b
    HV = w.HV
    err_da = np.abs(da.cpu().numpy() - rda)
    err_db = np.abs(db.cpu().numpy() - rdb)
    assert np.all(err_da <= 1e-4 * mdg * fac + 1e-6 * np.abs(rda).max()), float(err_da.max())
    assert np.all(err_db <= 1e-4 * mdb * bb + 1e-6 * np.abs(rdb).max()), float(err_db.max())
    bA = 1e-4 * mdg * np.abs(g64).reshape(-1, HV).sum(axis=0) + 1e-6 * np.abs(ref["dg"] * g64).reshape(-1, HV).sum(axis=0)
    bD = 1e-4 * mdg * fac.reshape(-1, HV).sum(axis=0) + 1e-6 * np.abs(rda).reshape(-1, HV).sum(axis=0)
    assert np.all(np.abs(dA.cpu().numpy() - rdA) <= bA) and np.all(np.abs(ddt.cpu().numpy() - rddt) <= bD)
    _say(f"    chain: max|da err| {float(err_da.max()):.2e} max|db err| {float(err_db.max()):.2e}")
