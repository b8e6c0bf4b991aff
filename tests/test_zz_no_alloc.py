"""The allocation-free forward entry point gdn_chunk_fwd_noalloc against
gdn_chunk_fwd given a workspace, both through the C ABI.

Two split calls in a row, the second on smaller sizes (so it runs over what
the first left in the static scratch), then a packed batch that needs no
scratch and one long sequence at the largest scratch use.  Both entry points run the same deterministic kernels, so their
results must be bitwise equal; each result is also held to the bf16 bars of
the split parity tests against the fp64 oracle (2e-2 on o, 1e-2 on the final
state).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
BARS = (2e-2, 1e-2)

CALLS = [
    # 8 segments of 576 tokens, the last 145
    ("first", scaled(WORKLOADS["gva"], "noalloc_first", B=1, T=4177, H=2, HV=4)),
    # smaller: 7 segments of 320 tokens, the last 180; K != V; no initial state
    ("second", scaled(WORKLOADS["gva"], "noalloc_second", B=2, T=2100, H=1, HV=2, K=64, V=128, init="none")),
]


def _gdn():
    import gated_deltanet_chunked_delta_amd as gdn
    gdn.load_library()
    return gdn


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _device_inputs(x):
    d = lambda t: None if t is None else t.to(DEV)
    q, k, v = (x[n].to(DEV, torch.bfloat16) for n in ("q", "k", "v"))
    return q, k, v, d(x["g"]), d(x["beta"]), d(x["initial_state"]), d(x["cu_seqlens"])


def _both(x):
    """(need, out and final state of gdn_chunk_fwd with a workspace, the same
    of gdn_chunk_fwd_noalloc)."""
    gdn = _gdn()
    q, k, v, g, beta, s0, cu = _device_inputs(x)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    N = x["N"]
    shape = gdn.make_shape(B, T, H, HV, K, V, N, gdn.GDN_BF16)
    need = gdn.gdn_chunk_fwd_workspace_bytes(shape) if cu is None else 0
    res = []
    for noalloc in (False, True):
        out = torch.full((B, T, HV, V), float("nan"), dtype=torch.bfloat16, device=DEV)
        fin = torch.full((N, HV, K, V), float("nan"), device=DEV)
        if noalloc:
            st = gdn.gdn_chunk_fwd_noalloc(q, k, v, g, beta, x["scale"], x["use_l2norm"], s0, cu, out, fin, shape)
        else:
            ws = torch.empty(need, dtype=torch.uint8, device=DEV) if need else None
            st = gdn.gdn_chunk_fwd(q, k, v, g, beta, x["scale"], x["use_l2norm"], s0, cu, out, fin, shape, ws)
        torch.cuda.synchronize()
        assert st == 0, gdn.gdn_status_str(st)
        res.append((out, fin))
    return need, res[0], res[1]


def _check_oracle(x, out, fin, label):
    o_ref, f_ref = oracle.recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"], scale=x["scale"],
                                    use_l2norm=x["use_l2norm"], initial_state=x["initial_state"],
                                    cu_seqlens=x["cu_seqlens"])
    eo = float(np.abs(out.float().cpu().numpy().astype(np.float64) - o_ref).max())
    ef = float(np.abs(fin.cpu().numpy().astype(np.float64) - f_ref).max())
    _say(f"[noalloc] {label}: max|do|={eo:.3e} (bar {BARS[0]})  max|dS|={ef:.3e} (bar {BARS[1]})")
    assert eo <= BARS[0] and ef <= BARS[1]


def test_noalloc_matches_workspace_entry_point_twice():
    gdn = _gdn()
    for i, (label, w) in enumerate(CALLS):
        _say(f"[noalloc] call {i}: {label} B={w.B} T={w.T} H={w.H} HV={w.HV} K={w.K} V={w.V}")
        x = oracle.add_gates(make_inputs(w, seed=41 + i, io_dtype=torch.float32))
        need, (o1, f1), (o2, f2) = _both(x)
        assert 0 < need <= gdn.GDN_STATIC_SCRATCH_BYTES, "these sizes are meant to use the scratch"
        assert torch.equal(o1, o2) and torch.equal(f1, f2), f"{label}: no-alloc result differs"
        _check_oracle(x, o2, f2, label)


def test_noalloc_without_split_and_long():
    gdn = _gdn()
    # a packed batch: no split, no scratch
    w = scaled(WORKLOADS["varlen"], "noalloc_packed", H=2, HV=4, lengths=(1, 300, 0, 65))
    x = oracle.add_gates(make_inputs(w, seed=43, io_dtype=torch.float32))
    _say("[noalloc] packed batch")
    need, (o1, f1), (o2, f2) = _both(x)
    assert need == 0
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    _check_oracle(x, o2, f2, "packed")
    # one long sequence at the long workload's head count (8 segments of 2048,
    # the static scratch's largest use), against the workspace entry point
    w = scaled(WORKLOADS["long"], "noalloc_long", T=16384)
    x = make_inputs(w, seed=44, device="cuda:0")
    g, beta = gdn.fused_gdn_gating(x["A_log"], x["a"], x["b"], x["dt_bias"])
    x["g"], x["beta"] = g, beta
    _say("[noalloc] one sequence of 16384 tokens, 32 value heads")
    need, (o1, f1), (o2, f2) = _both(x)
    assert 0 < need <= gdn.GDN_STATIC_SCRATCH_BYTES
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    assert torch.isfinite(o2).all() and torch.isfinite(f2).all()


def test_noalloc_graph_capture():
    """The call the entry point exists for: captured into a HIP graph (no
    allocation, no memory fill inside), replayed three times, with another
    split call of other sizes overwriting the static scratch between the
    replays; every replay equals the eager call bit for bit."""
    gdn = _gdn()
    w = CALLS[0][1]
    x = oracle.add_gates(make_inputs(w, seed=45, io_dtype=torch.float32))
    q, k, v, g, beta, s0, cu = _device_inputs(x)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    shape = gdn.make_shape(B, T, H, HV, K, V, B, gdn.GDN_BF16)
    assert gdn.gdn_chunk_fwd_workspace_bytes(shape) > 0
    out = torch.empty((B, T, HV, V), dtype=torch.bfloat16, device=DEV)
    fin = torch.empty((B, HV, K, V), device=DEV)

    def call():
        st = gdn.gdn_chunk_fwd_noalloc(q, k, v, g, beta, x["scale"], x["use_l2norm"], s0, cu, out, fin, shape)
        assert st == 0, gdn.gdn_status_str(st)

    call()
    torch.cuda.synchronize()
    ref_o, ref_f = out.clone(), fin.clone()
    # the other split call that overwrites the scratch between replays
    x2 = oracle.add_gates(make_inputs(CALLS[1][1], seed=46, io_dtype=torch.float32))
    q2, k2, v2, g2, b2, s02, _ = _device_inputs(x2)
    B2, T2, H2, K2 = q2.shape
    HV2, V2 = v2.shape[2], v2.shape[3]
    shape2 = gdn.make_shape(B2, T2, H2, HV2, K2, V2, B2, gdn.GDN_BF16)
    out2 = torch.empty((B2, T2, HV2, V2), dtype=torch.bfloat16, device=DEV)
    fin2 = torch.empty((B2, HV2, K2, V2), device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up off the default stream before capture
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(7)
        fin.fill_(7)
        st = gdn.gdn_chunk_fwd_noalloc(q2, k2, v2, g2, b2, x2["scale"], x2["use_l2norm"], s02, None, out2, fin2,
                                       shape2)
        assert st == 0
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(fin, ref_f), f"replay {i} differs from the eager call"
    _say("[noalloc] graph: 3 replays equal to the eager call")
