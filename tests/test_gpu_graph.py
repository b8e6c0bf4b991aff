"""HIP graph capture of the library's calls, as a serving or training loop
would use them: each call is captured once into a torch.cuda.CUDAGraph and
replayed several times, with eager work and synchronisations between the
replays.  The outputs are overwritten with a sentinel before every replay and
every replay must reproduce the eager call bit for bit (the same kernels on the
same inputs; the arithmetic is deterministic).  Calls that update state in
place get their state restored, outside the graph, before each replay.
"""
import sys

import pytest
import torch

import oracle
from workloads import WORKLOADS, make_grad_inputs, make_inputs, scaled

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
REPLAYS = 3


def _gdn():
    import gated_deltanet_chunked_delta_amd as gdn
    gdn.load_library()
    return gdn


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check_graph(name, fn, reset=lambda: None):
    """fn() issues the library call(s) on the current stream and returns the
    output tensors; reset() restores whatever the call updates in place."""
    reset()
    ref = [t.clone() for t in fn()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up off the default stream before capture
        reset()
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = fn()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        for t in outs:
            t.fill_(7)
        reset()   # after the sentinel: a state updated in place is input and output
        busy = torch.randn(1 << 20, device=DEV)   # unrelated eager work between replays
        busy.mul_(2.0).sum().item()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j, (got, want) in enumerate(zip(outs, ref)):
            assert torch.equal(got, want), f"{name}: replay {i}, output {j} differs from the eager call"
    _say(f"    {name}: {REPLAYS} replays equal to the eager call")


def _fwd_inputs(w, seed):
    x = oracle.add_gates(make_inputs(w, seed=seed, io_dtype=torch.float32))
    to = lambda t, dt=None: None if t is None else t.to(DEV, dt) if dt else t.to(DEV)
    return x, {"q": to(x["q"], torch.bfloat16), "k": to(x["k"], torch.bfloat16),
               "v": to(x["v"], torch.bfloat16), "g": to(x["g"]), "beta": to(x["beta"]),
               "h0": to(x["initial_state"]), "cu": to(x["cu_seqlens"])}


@pytest.mark.parametrize("name", ["gva_ragged", "varlen_mix", "split_long"])
def test_graph_prefill(name):
    gdn = _gdn()
    w = {"gva_ragged": scaled(WORKLOADS["gva"], "gva_ragged", B=2, T=300, H=2, HV=4),
         "varlen_mix": scaled(WORKLOADS["varlen"], "varlen_mix", H=2, HV=4, lengths=(1, 64, 65, 0, 200, 3)),
         # few long sequences: the call runs the sequence split (five kernels) in the workspace
         "split_long": scaled(WORKLOADS["gva"], "split_long", B=1, T=2048, H=1, HV=2)}[name]
    x, d = _fwd_inputs(w, seed=41)
    B, T, H, K = d["q"].shape
    shape = gdn.make_shape(B, T, H, w.HV, K, w.V, x["N"], gdn.GDN_BF16)
    need = gdn.gdn_chunk_fwd_workspace_bytes(shape)
    # the split runs its five kernels in the workspace; a packed batch keeps the
    # longest-first order of its sequences there (one kernel before the prefill)
    assert (need > 0) == (name in ("split_long", "varlen_mix"))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    _say(f"[graph] prefill {name}: workspace {need} bytes")

    def fn():
        o, ht = gdn.chunk_gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=x["scale"],
                                           initial_state=d["h0"], cu_seqlens=d["cu"],
                                           use_qk_l2norm_in_kernel=x["use_l2norm"], workspace=ws)
        return [o, ht]
    _check_graph(f"prefill {name}", fn)


def test_graph_decode_pool():
    gdn = _gdn()
    torch.manual_seed(5)
    N, H, HV, K, V, P = 24, 2, 4, 128, 128, 40
    q = torch.randn(N, H, K, device=DEV, dtype=torch.bfloat16)
    k = torch.randn(N, H, K, device=DEV, dtype=torch.bfloat16)
    v = torch.randn(N, HV, V, device=DEV, dtype=torch.bfloat16)
    g = -torch.rand(N, HV, device=DEV)
    beta = torch.rand(N, HV, device=DEV)
    idx = torch.randperm(P, device=DEV)[:N].to(torch.int32)
    idx[3] = -1                                    # a padding row
    pool0 = 0.05 * torch.randn(P, HV, K, V, device=DEV)
    pool = pool0.clone()
    out = torch.empty(N, HV, V, device=DEV, dtype=torch.bfloat16)
    _say("[graph] decode with an in-place fp32 pool")

    def fn():
        gdn.fused_recurrent_gated_delta_rule_update(q, k, v, g, beta, pool, idx, use_qk_l2norm_in_kernel=True,
                                                     out=out)
        return [out, pool]
    _check_graph("decode", fn, reset=lambda: pool.copy_(pool0))


def test_graph_backward_and_gating():
    gdn = _gdn()
    w = scaled(WORKLOADS["gva"], "gva_ragged", B=2, T=300, H=2, HV=4)
    x = make_grad_inputs(oracle.add_gates(make_inputs(w, seed=43, io_dtype=torch.float32)), seed=143)
    bf = lambda t: t.to(DEV, torch.bfloat16)
    q, k, v, do = bf(x["q"]), bf(x["k"]), bf(x["v"]), bf(x["do"])
    g, beta, dht, h0 = (x[n].to(DEV) for n in ("g", "beta", "dht", "initial_state"))
    A_log, dt_bias = x["A_log"].to(DEV), x["dt_bias"].to(DEV)
    a, b = bf(x["a"]), bf(x["b"])
    _say("[graph] backward, gating and gate-input gradients")

    def fn():
        gg, bb = gdn.fused_gdn_gating(A_log, a, b, dt_bias)
        grads = gdn.chunk_gated_delta_rule_bwd(q, k, v, g, beta, do, dht=dht, scale=x["scale"], initial_state=h0,
                                               use_qk_l2norm_in_kernel=x["use_l2norm"])
        dgate = gdn.fused_gdn_gating_bwd(A_log, a, b, dt_bias, grads[3], grads[4])
        return [gg, bb, *grads, *dgate]
    _check_graph("backward + gating", fn)
