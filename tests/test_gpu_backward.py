"""GPU parity of the backward pass (gdn_chunk_bwd through the C ABI) against
the fp64 backward oracle (oracle/backward.py, pinned to finite differences).

Bars, as max|gpu - oracle| / max|oracle| per output: the kernels compute in
fp32 whatever the I/O type (fp32 products, or bf16 hi/lo splits of fp32
operands that keep about 16 bits of each product), so fp32 outputs (dg, dbeta,
dh0, and everything in the fp32 check mode) carry only fp32-level rounding: 1e-4.  bf16 outputs (dq, dk,
dv) are additionally rounded to bf16 once: half an ulp, at most 2^-8 of the
element (an element just above a power of two), so their bar is 2^-8 + 1e-4.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle.backward import backward as oracle_backward
from workloads import WORKLOADS, make_grad_inputs, make_inputs, scaled

pytestmark = pytest.mark.gpu

F32_BAR = 1e-4
BF16_BAR = 2.0 ** -8 + F32_BAR
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def _gdn():
    import gated_deltanet_chunked_delta_amd as gdn
    gdn.load_library()
    return gdn


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bars(dtype):
    lo = BF16_BAR if dtype == torch.bfloat16 else F32_BAR
    return {"dq": lo, "dk": lo, "dv": lo, "dg": F32_BAR, "dbeta": F32_BAR, "dh0": F32_BAR}


def run_gpu_bwd(x, dtype, dht=True, init=True):
    gdn = _gdn()
    dev = torch.device("cuda:0")
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].to(dev)
    s0 = None if (x["initial_state"] is None or not init) else x["initial_state"].to(dev)
    out = gdn.chunk_gated_delta_rule_bwd(
        x["q"].to(dev, dtype), x["k"].to(dev, dtype), x["v"].to(dev, dtype), x["g"].to(dev), x["beta"].to(dev),
        x["do"].to(dev, dtype), dht=x["dht"].to(dev) if dht else None, scale=x["scale"], initial_state=s0,
        cu_seqlens=cu, use_qk_l2norm_in_kernel=x["use_l2norm"])
    torch.cuda.synchronize()
    return dict(zip(NAMES, out))


def run_oracle_bwd(x, dht=True, init=True):
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].cpu().numpy()
    return oracle_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"],
                           dht=x["dht"] if dht else None, scale=x["scale"], use_l2norm=x["use_l2norm"],
                           initial_state=x["initial_state"] if init else None, cu_seqlens=cu)


def compare(got, ref, bars, tag):
    worst = {}
    for name in NAMES:
        g = got[name].float().cpu().numpy().astype(np.float64)
        r = ref[name]
        if r.size == 0:
            continue
        m = float(np.abs(r).max())
        err = float(np.abs(g - r).max()) / max(m, 1e-30)
        worst[name] = err
        _say(f"    {tag} {name}: rel max err {err:.2e} (bar {bars[name]:.1e}, max|ref| {m:.3e})")
    for name, err in worst.items():
        assert err <= bars[name], f"{tag}: {name} relative error {err} > {bars[name]}"


SMALL = {
    "tiny": WORKLOADS["tiny"],
    "gva_ragged": scaled(WORKLOADS["gva"], "gva_ragged", B=2, T=300, H=2, HV=4),
    "varlen_mix": scaled(WORKLOADS["varlen"], "varlen_mix", H=2, HV=4,
                         lengths=(1, 64, 65, 127, 0, 200, 3, 129)),
    "long_slow": scaled(WORKLOADS["long"], "long_slow", T=700, H=1, HV=2),
    "wide_small": scaled(WORKLOADS["wide_stable"], "wide_small", B=3, T=257, H=2, HV=4),
    "k64_v128": scaled(WORKLOADS["gva"], "k64_v128", B=2, T=190, H=2, HV=4, K=64, V=128),
    "k128_v64": scaled(WORKLOADS["gva"], "k128_v64", B=2, T=130, H=1, HV=3, K=128, V=64),
    "four_per_key_head": scaled(WORKLOADS["gva"], "four_per_key_head", B=1, T=200, H=2, HV=8),
    # the scans' tile width follows the (sequence, value head) count: 3 x 16 heads
    # take 32-column tiles, 5 x 16 the 64-column ones (the cases above, 16-column)
    "mid_width_tiles": scaled(WORKLOADS["gva"], "mid_width_tiles", B=3, T=200, H=8, HV=16),
    "wide_tiles": scaled(WORKLOADS["gva"], "wide_tiles", B=5, T=130, H=8, HV=16),
    # the same tile widths with K = 64 (the K = 64 variants of both scans): (sequence,
    # value head, 64-column) units 96 and 160 with V = 128, 80 and 160 with V = 64
    "mid_width_tiles_k64": scaled(WORKLOADS["gva"], "mid_width_tiles_k64", B=3, T=200, H=8, HV=16, K=64),
    "wide_tiles_k64": scaled(WORKLOADS["gva"], "wide_tiles_k64", B=5, T=130, H=8, HV=16, K=64),
    "mid_width_tiles_k64_v64": scaled(WORKLOADS["gva"], "mid_width_tiles_k64_v64", B=5, T=150, H=8, HV=16,
                                      K=64, V=64),
    "wide_tiles_k64_v64": scaled(WORKLOADS["gva"], "wide_tiles_k64_v64", B=10, T=100, H=8, HV=16, K=64, V=64),
}


def _inputs(w, seed=0):
    x = oracle.add_gates(make_inputs(w, seed=seed, io_dtype=torch.float32))
    return make_grad_inputs(x, seed=seed + 100)


@pytest.mark.parametrize("n_seqs", [1024, 1025])
def test_backward_packed_order_is_position_neutral(n_seqs):
    """The scans take packed sequences longest first (up to 1024 sequences,
    ranked by the setup kernel); a sequence's gradients do not depend on which
    workgroup computes it or where it sits in the batch: the batch and the
    same sequences in reverse order give bitwise equal gradients per sequence."""
    rng = np.random.default_rng(n_seqs)
    lens = [int(x) for x in rng.integers(0, 25, n_seqs)]
    w = scaled(WORKLOADS["varlen"], f"bwd_many_{n_seqs}", H=2, HV=4, K=64, V=64, lengths=tuple(lens))
    x = make_grad_inputs(oracle.add_gates(make_inputs(w, seed=9, io_dtype=torch.float32)), seed=10)
    starts = np.concatenate([[0], np.cumsum(lens)])
    perm = list(range(n_seqs))[::-1]
    tok = np.concatenate([np.arange(starts[n], starts[n + 1]) for n in perm]).astype(np.int64)
    xr = dict(x)
    for name in ("q", "k", "v", "g", "beta", "do"):
        xr[name] = x[name][:, tok]
    for name in ("initial_state", "dht"):
        if x[name] is not None:
            xr[name] = x[name][perm]
    xr["cu_seqlens"] = torch.tensor(np.concatenate([[0], np.cumsum([lens[n] for n in perm])]), dtype=torch.int32)
    a = run_gpu_bwd(x, torch.bfloat16)
    b = run_gpu_bwd(xr, torch.bfloat16)
    back = np.argsort(tok)
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        assert torch.equal(a[name], b[name][:, torch.as_tensor(back, device=b[name].device)]), name
    assert torch.equal(a["dh0"], b["dh0"][torch.as_tensor(perm, device=b["dh0"].device)])
    _say(f"[bwd order] {n_seqs} sequences: gradients equal under reversal")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("name", list(SMALL))
def test_backward_small(name, dtype):
    x = _inputs(SMALL[name])
    _say(f"[bwd] {name} dtype={dtype} lens={x['lens'][:8]}")
    got = run_gpu_bwd(x, dtype)
    ref = run_oracle_bwd(x)
    compare(got, ref, _bars(dtype), name)


def test_backward_without_state_gradients():
    """No initial state and no final-state gradient."""
    x = _inputs(SMALL["gva_ragged"], seed=3)
    _say("[bwd] gva_ragged without initial state / dht")
    got = run_gpu_bwd(x, torch.bfloat16, dht=False, init=False)
    ref = run_oracle_bwd(x, dht=False, init=False)
    compare(got, ref, _bars(torch.bfloat16), "no-state")


def test_backward_deterministic_bitwise():
    x = _inputs(SMALL["varlen_mix"], seed=4)
    a = run_gpu_bwd(x, torch.bfloat16)
    b = run_gpu_bwd(x, torch.bfloat16)
    for name in NAMES:
        assert torch.equal(a[name], b[name]), name


def test_backward_empty_sequences():
    """Zero-length sequences: no token gradients; dh0 = dht."""
    w = scaled(WORKLOADS["varlen"], "empty", H=2, HV=4, lengths=(0, 0, 0))
    x = _inputs(w, seed=6)
    got = run_gpu_bwd(x, torch.bfloat16)
    assert got["dq"].numel() == 0 and got["dv"].numel() == 0
    assert torch.equal(got["dh0"].cpu(), x["dht"])


def test_backward_gva_full_size_sampled():
    """The 4 x 4096-token, 32-value-head workload at full size, in the
    configuration the benchmark times; key-head groups sampled against the
    oracle (both value heads of each group, so dq and dk are complete)."""
    w = WORKLOADS["gva"]
    _say("[bwd-full] gva: generating on the GPU")
    x = make_grad_inputs(oracle.add_gates(make_inputs(w, seed=0, device="cuda:0")), seed=100)
    got = run_gpu_bwd(x, torch.bfloat16)
    for name in NAMES:
        assert torch.isfinite(got[name]).all(), name
    G = w.HV // w.H
    bars = _bars(torch.bfloat16)
    for n, jk in ((0, 0), (3, w.H - 1), (2, 7)):
        sl = slice(jk * G, (jk + 1) * G)
        sub = dict(q=x["q"][n:n + 1, :, jk:jk + 1].cpu(), k=x["k"][n:n + 1, :, jk:jk + 1].cpu(),
                   v=x["v"][n:n + 1, :, sl].cpu(), g=x["g"][n:n + 1, :, sl].cpu(),
                   beta=x["beta"][n:n + 1, :, sl].cpu(), do=x["do"][n:n + 1, :, sl].cpu(),
                   dht=x["dht"][n:n + 1, sl].cpu(),
                   initial_state=None if x["initial_state"] is None else x["initial_state"][n:n + 1, sl].cpu(),
                   cu_seqlens=None, scale=x["scale"], use_l2norm=x["use_l2norm"])
        ref = run_oracle_bwd(sub)
        part = {"dq": got["dq"][n:n + 1, :, jk:jk + 1], "dk": got["dk"][n:n + 1, :, jk:jk + 1],
                "dv": got["dv"][n:n + 1, :, sl], "dg": got["dg"][n:n + 1, :, sl],
                "dbeta": got["dbeta"][n:n + 1, :, sl], "dh0": got["dh0"][n:n + 1, sl]}
        compare(part, ref, bars, f"gva n={n} key head {jk}")


def test_backward_varlen_full_size_sampled():
    """The packed 64-sequence workload (about 65k tokens, lengths 1..2048) at full
    size, as one call; sampled (sequence, key head) groups, with both value heads
    of each group, against the oracle: the longest sequence, the first and the
    last, at the first, a middle and the last key head."""
    w = WORKLOADS["varlen"]
    _say("[bwd-full] varlen: generating on the GPU")
    x = make_grad_inputs(oracle.add_gates(make_inputs(w, seed=0, device="cuda:0")), seed=100)
    got = run_gpu_bwd(x, torch.bfloat16)
    for name in NAMES:
        assert torch.isfinite(got[name]).all(), name
    G = w.HV // w.H
    bars = _bars(torch.bfloat16)
    starts = [int(c) for c in x["cu_seqlens"].tolist()]
    N = x["N"]
    longest = int(np.argmax(x["lens"]))
    for n, jk in ((0, 0), (longest, w.H // 2), (N - 1, w.H - 1)):
        t0, t1 = starts[n], starts[n + 1]
        sl = slice(jk * G, (jk + 1) * G)

        def rows(t, heads):
            return t[0, t0:t1, heads].unsqueeze(0).cpu()
        sub = dict(q=rows(x["q"], slice(jk, jk + 1)), k=rows(x["k"], slice(jk, jk + 1)), v=rows(x["v"], sl),
                   g=rows(x["g"], sl), beta=rows(x["beta"], sl), do=rows(x["do"], sl),
                   dht=x["dht"][n:n + 1, sl].cpu(),
                   initial_state=None if x["initial_state"] is None else x["initial_state"][n:n + 1, sl].cpu(),
                   cu_seqlens=None, scale=x["scale"], use_l2norm=x["use_l2norm"])
        _say(f"    group n={n} len={t1 - t0} key head {jk}")
        ref = run_oracle_bwd(sub)
        part = {"dq": got["dq"][0:1, t0:t1, jk:jk + 1], "dk": got["dk"][0:1, t0:t1, jk:jk + 1],
                "dv": got["dv"][0:1, t0:t1, sl], "dg": got["dg"][0:1, t0:t1, sl],
                "dbeta": got["dbeta"][0:1, t0:t1, sl], "dh0": got["dh0"][n:n + 1, sl]}
        compare(part, ref, bars, f"varlen n={n} key head {jk}")


def test_backward_wide_full_size_sampled():
    """The largest workload at full size (16 x 16384 tokens, 64 value heads, no L2
    norm, the parity inputs of the wide workload): workspace offsets past 2^32
    elements, 4096 chunks per value head; sampled (sequence, key head) groups,
    both value heads each, against the oracle."""
    w = WORKLOADS["wide_stable"]
    _say("[bwd-full] wide: generating on the GPU")
    x = make_grad_inputs(oracle.add_gates(make_inputs(w, seed=0, device="cuda:0")), seed=100)
    got = run_gpu_bwd(x, torch.bfloat16)
    for name in NAMES:
        assert torch.isfinite(got[name]).all(), name
    G = w.HV // w.H
    bars = _bars(torch.bfloat16)
    for n, jk in ((0, 0), (w.B - 1, w.H - 1), (7, 13)):
        sl = slice(jk * G, (jk + 1) * G)
        sub = dict(q=x["q"][n:n + 1, :, jk:jk + 1].cpu(), k=x["k"][n:n + 1, :, jk:jk + 1].cpu(),
                   v=x["v"][n:n + 1, :, sl].cpu(), g=x["g"][n:n + 1, :, sl].cpu(),
                   beta=x["beta"][n:n + 1, :, sl].cpu(), do=x["do"][n:n + 1, :, sl].cpu(),
                   dht=x["dht"][n:n + 1, sl].cpu(),
                   initial_state=None if x["initial_state"] is None else x["initial_state"][n:n + 1, sl].cpu(),
                   cu_seqlens=None, scale=x["scale"], use_l2norm=x["use_l2norm"])
        _say(f"    group n={n} key head {jk}")
        ref = run_oracle_bwd(sub)
        part = {"dq": got["dq"][n:n + 1, :, jk:jk + 1], "dk": got["dk"][n:n + 1, :, jk:jk + 1],
                "dv": got["dv"][n:n + 1, :, sl], "dg": got["dg"][n:n + 1, :, sl],
                "dbeta": got["dbeta"][n:n + 1, :, sl], "dh0": got["dh0"][n:n + 1, sl]}
        compare(part, ref, bars, f"wide n={n} key head {jk}")


def test_backward_long_full_size_sampled():
    """One 131,072-token sequence with slow decay (2048 chunks through the
    scans' narrowest, 16-column tiles): one key head, both its value heads,
    against the oracle over the whole sequence."""
    w = WORKLOADS["long"]
    _say("[bwd-full] long: generating on the GPU")
    x = make_grad_inputs(oracle.add_gates(make_inputs(w, seed=0, device="cuda:0")), seed=100)
    got = run_gpu_bwd(x, torch.bfloat16)
    for name in NAMES:
        assert torch.isfinite(got[name]).all(), name
    G = w.HV // w.H
    jk = w.H // 2
    sl = slice(jk * G, (jk + 1) * G)
    sub = dict(q=x["q"][:, :, jk:jk + 1].cpu(), k=x["k"][:, :, jk:jk + 1].cpu(), v=x["v"][:, :, sl].cpu(),
               g=x["g"][:, :, sl].cpu(), beta=x["beta"][:, :, sl].cpu(), do=x["do"][:, :, sl].cpu(),
               dht=x["dht"][:, sl].cpu(),
               initial_state=None if x["initial_state"] is None else x["initial_state"][:, sl].cpu(),
               cu_seqlens=None, scale=x["scale"], use_l2norm=x["use_l2norm"])
    _say(f"    key head {jk}: the oracle over {w.T} tokens")
    ref = run_oracle_bwd(sub)
    part = {"dq": got["dq"][:, :, jk:jk + 1], "dk": got["dk"][:, :, jk:jk + 1], "dv": got["dv"][:, :, sl],
            "dg": got["dg"][:, :, sl], "dbeta": got["dbeta"][:, :, sl], "dh0": got["dh0"][:, sl]}
    compare(part, ref, _bars(torch.bfloat16), f"long key head {jk}")
