"""GPU parity of the sequence split (few long equal-length sequences cut into
segments that run side by side, chained through their transfer maps) against
the fp64 oracle, through the C ABI; and split against unsplit.

Bars as for prefill: bf16 inputs 2e-2 on o and 1e-2 on the final state, fp32
check mode 1e-4.  The split path runs when the caller passes the workspace
gdn_chunk_fwd_workspace_bytes asks for (the Python binding does); without it
the same call runs unsplit.
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


CASES = {
    # 4 workgroups unsplit -> 8 segments of 256 tokens
    "even": scaled(WORKLOADS["gva"], "split_even", B=1, T=2048, H=1, HV=2),
    # ragged last segment (7 segments of 320, the last 180), K != V, no initial state
    "ragged_k64": scaled(WORKLOADS["gva"], "split_ragged", B=2, T=2100, H=1, HV=2, K=64, V=128, init="none"),
    "k128_v64": scaled(WORKLOADS["gva"], "split_v64", B=1, T=3000, H=2, HV=4, K=128, V=64),
    "slow_decay": scaled(WORKLOADS["long"], "split_long", T=4096, H=1, HV=2),
    # 64 workgroups unsplit -> 8 segments of 1152 tokens (the last 936), run
    # as whole 128-column value heads; the combine chains 32 value heads x 4
    # column blocks through seven transfer maps
    "multi_block": scaled(WORKLOADS["gva"], "split_multi_block", B=1, T=9000, H=16, HV=32),
}


def _run(x, dtype, split=True, gated=False, final=True):
    gdn = _gdn()
    d = lambda t: None if t is None else t.to(DEV)
    q, k, v = (x[n].to(DEV, dtype) for n in ("q", "k", "v"))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    shape = gdn.make_shape(B, T, H, HV, K, V, B, gdn.GDN_BF16 if dtype == torch.bfloat16 else gdn.GDN_F32)
    need = gdn.gdn_chunk_fwd_workspace_bytes(shape)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV) if (split and need) else None
    out = torch.empty((B, T, HV, V), dtype=dtype, device=DEV)
    fin = torch.empty((B, HV, K, V), device=DEV) if final else None
    s0 = d(x["initial_state"])
    if gated:
        a, b = x["a"].to(DEV, dtype), x["b"].to(DEV, dtype)
        gates = gdn.make_gates(d(x["A_log"]), d(x["dt_bias"]), a, b)
        st = gdn.gdn_chunk_fwd_gated(q, k, v, gates, x["scale"], x["use_l2norm"], s0, None, out, fin, shape, ws)
    else:
        st = gdn.gdn_chunk_fwd(q, k, v, d(x["g"]), d(x["beta"]), x["scale"], x["use_l2norm"], s0, None, out, fin,
                               shape, ws)
    torch.cuda.synchronize()
    assert st == 0, gdn.gdn_status_str(st)
    return need, out, fin


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("name", list(CASES))
def test_split_parity(name, dtype):
    w = CASES[name]
    x = oracle.add_gates(make_inputs(w, seed=31, io_dtype=torch.float32))
    need, o, fin = _run(x, dtype)
    assert need > 0, "these sizes are meant to be split"
    o_ref, f_ref = oracle.recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"], scale=x["scale"],
                                    use_l2norm=x["use_l2norm"], initial_state=x["initial_state"])
    eo = float(np.abs(o.float().cpu().numpy().astype(np.float64) - o_ref).max())
    ef = float(np.abs(fin.cpu().numpy().astype(np.float64) - f_ref).max())
    to, tf = TOL[dtype]
    _say(f"[split] {name} {dtype}: workspace {need / 2**20:.1f} MiB  max|do|={eo:.3e} (bar {to})  "
         f"max|dS|={ef:.3e} (bar {tf})")
    assert eo <= to and ef <= tf


def test_split_matches_unsplit_and_gated():
    w = CASES["even"]
    x = make_inputs(w, seed=32)
    oracle.add_gates(x)
    _, o1, f1 = _run(x, torch.bfloat16, split=True)
    _, o2, f2 = _run(x, torch.bfloat16, split=False)
    do, df = float((o1.float() - o2.float()).abs().max()), float((f1 - f2).abs().max())
    _say(f"    split vs unsplit: max|do|={do:.3e} max|dS|={df:.3e}")
    assert do <= 2e-2 and df <= 1e-2
    # in-kernel gating through the split path, and no final state requested
    _, o3, _ = _run(x, torch.bfloat16, split=True, gated=True, final=False)
    o_ref, _ = oracle.recurrent_gated(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"], x["b"],
                                      scale=x["scale"], use_l2norm=True, initial_state=x["initial_state"])
    eo = float(np.abs(o3.float().cpu().numpy().astype(np.float64) - o_ref).max())
    _say(f"    gated split: max|do|={eo:.3e}")
    assert eo <= 2e-2
