"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars (max-abs error against the oracle): bf16 inputs -> 2e-2 on o and 1e-2 on
the final state; fp32 check mode -> 1e-4 on both.  bf16 runs also meet
regression bars relative to the size of the result (2 % of max|o|, 1.5 % of
max|S|; the kernel measures at most 0.6 % and 0.5 %), and the discriminating
cases of ``parity_cases`` meet their own bars, which every planted mistake
misses by at least a factor of five (``test_parity_gate_power``).  Small cases
run the whole oracle; the full-size workloads compare sampled (sequence, value
head) units, in the same launch configuration the benchmark times, in bf16 and
in the fp32 check mode.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import parity_cases
from workloads import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: (2e-2, 1e-2), torch.float32: (1e-4, 1e-4)}
REL_BF16 = (0.02, 0.015)   # regression bars of bf16 runs, relative to max|o|, max|S| of the oracle


def _gdn():
    import gated_deltanet_chunked_delta_amd as gdn
    gdn.load_library()
    return gdn


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(x, dtype=None, **kw):
    gdn = _gdn()
    dev = torch.device("cuda:0")
    d = dtype or x["q"].dtype
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].to(dev)
    s0 = None if x["initial_state"] is None else x["initial_state"].to(dev)
    o, fin = gdn.chunk_gated_delta_rule(x["q"].to(dev, d), x["k"].to(dev, d), x["v"].to(dev, d),
                                        x["g"].to(dev), x["beta"].to(dev), scale=x["scale"],
                                        initial_state=s0, cu_seqlens=cu,
                                        use_qk_l2norm_in_kernel=x["use_l2norm"], **kw)
    torch.cuda.synchronize()
    return o, fin


def oracle_full(x):
    return oracle.recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"], scale=x["scale"],
                            use_l2norm=x["use_l2norm"], initial_state=x["initial_state"],
                            cu_seqlens=None if x["cu_seqlens"] is None else x["cu_seqlens"].cpu().numpy())


def check_errors(eo, ef, o_ref, f_ref, dtype, bars=None):
    """Asserts the bars on the max-abs errors eo (outputs) and ef (final states)."""
    to, tf = bars or TOL[dtype]
    mo = float(np.abs(o_ref).max()) if np.size(o_ref) else 0.0
    mf = float(np.abs(f_ref).max()) if np.size(f_ref) else 0.0
    _say(f"    max|do|={eo:.3e} (bar {to}, {eo / max(mo, 1e-30):.2%} of max|o|)  "
         f"max|dS|={ef:.3e} (bar {tf}, {ef / max(mf, 1e-30):.2%} of max|S|)")
    assert eo <= to and ef <= tf
    if dtype == torch.bfloat16:
        assert eo <= REL_BF16[0] * mo and ef <= REL_BF16[1] * mf, "bf16 regression bar"


def check_full(x, dtype, bars=None):
    _say(f"[parity] {x['workload'].name} dtype={dtype} lens={x['lens'][:8]}")
    o, fin = run_gpu(x, dtype)
    o_ref, f_ref = oracle_full(x)
    eo = float(np.abs(o.float().cpu().numpy().astype(np.float64) - o_ref).max()) if o.numel() else 0.0
    ef = float(np.abs(fin.cpu().numpy().astype(np.float64) - f_ref).max()) if fin.numel() else 0.0
    check_errors(eo, ef, o_ref, f_ref, dtype, bars)
    return eo, ef


SMALL = {
    "tiny": WORKLOADS["tiny"],
    "gva_ragged": scaled(WORKLOADS["gva"], "gva_ragged", B=2, T=300, H=2, HV=4),
    "varlen_mix": scaled(WORKLOADS["varlen"], "varlen_mix", H=2, HV=4,
                         lengths=(1, 64, 65, 127, 0, 200, 3, 129)),
    "long_slow": scaled(WORKLOADS["long"], "long_slow", T=1000, H=1, HV=2),
    "wide_stable": scaled(WORKLOADS["wide_stable"], "wide_small", B=3, T=257, H=2, HV=4),
    "k64_v128": scaled(WORKLOADS["gva"], "k64_v128", B=2, T=190, H=2, HV=4, K=64, V=128),
    "k128_v64": scaled(WORKLOADS["gva"], "k128_v64", B=2, T=130, H=1, HV=3, K=128, V=64),
    # at least 256 (sequence, value head) pairs: whole 128-column value heads per workgroup
    "heads_ragged": scaled(WORKLOADS["gva"], "heads_ragged", B=2, T=200, H=8, HV=128),
    "heads_varlen": scaled(WORKLOADS["varlen"], "heads_varlen", H=16, HV=32,
                           lengths=(1, 64, 65, 127, 0, 200, 3, 129)),
    "heads_k64": scaled(WORKLOADS["gva"], "heads_k64", B=4, T=100, H=16, HV=64, K=64, V=128),
    # the same layout without the L2 norm (its P tiles are formed by chain waves)
    "heads_nonorm": scaled(WORKLOADS["wide_stable"], "heads_nonorm", B=2, T=200, H=8, HV=128),
    "heads_nonorm_k64": scaled(WORKLOADS["wide_stable"], "heads_nonorm_k64", B=4, T=100, H=16, HV=64, K=64,
                               V=128, qk_std=64 ** -0.5),
    "heads_nonorm_varlen": scaled(WORKLOADS["varlen"], "heads_nonorm_varlen", H=16, HV=32, use_l2norm=False,
                                  qk_std=128 ** -0.5, lengths=(1, 64, 65, 127, 0, 200, 3, 129)),
}


# the 128-column layout exists for bf16 only (the fp32 check mode has one layout)
BF16_ONLY = {"heads_ragged", "heads_varlen", "heads_k64", "heads_nonorm", "heads_nonorm_k64", "heads_nonorm_varlen"}


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("name", list(SMALL))
def test_parity_small(name, dtype):
    if dtype == torch.float32 and name in BF16_ONLY:
        pytest.skip("bf16 layout case")
    x = oracle.add_gates(make_inputs(SMALL[name], seed=0, io_dtype=torch.float32))
    check_full(x, dtype)


@pytest.mark.parametrize("name", list(parity_cases.cases()))
def test_parity_discriminating(name):
    """bf16 on inputs where every planted mistake misses the case's bars by 5x."""
    w, bar_o, bar_s = parity_cases.cases()[name]
    x = oracle.add_gates(make_inputs(w, seed=0, io_dtype=torch.float32))
    check_full(x, torch.bfloat16, bars=(bar_o, bar_s))


def test_final_state_aliases_initial_state():
    x = oracle.add_gates(make_inputs(SMALL["gva_ragged"], seed=1, io_dtype=torch.float32))
    gdn = _gdn()
    dev = torch.device("cuda:0")
    s = x["initial_state"].to(dev).clone()
    o, fin = gdn.chunk_gated_delta_rule(x["q"].to(dev, torch.bfloat16), x["k"].to(dev, torch.bfloat16),
                                        x["v"].to(dev, torch.bfloat16), x["g"].to(dev), x["beta"].to(dev),
                                        scale=x["scale"], initial_state=s, final_state=s,
                                        use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    o2, fin2 = run_gpu(x, torch.bfloat16)
    assert fin.data_ptr() == s.data_ptr()
    assert torch.equal(o, o2) and torch.equal(s, fin2)


def test_no_final_state_and_no_initial_state():
    x = oracle.add_gates(make_inputs(SMALL["tiny"], seed=2, io_dtype=torch.float32))
    o, fin = run_gpu(x, torch.bfloat16, output_final_state=False)
    assert fin is None
    o_ref, _ = oracle_full(x)
    assert float(np.abs(o.float().cpu().numpy() - o_ref).max()) <= 2e-2


def test_deterministic_bitwise():
    x = oracle.add_gates(make_inputs(SMALL["varlen_mix"], seed=3, io_dtype=torch.float32))
    o1, f1 = run_gpu(x, torch.bfloat16)
    o2, f2 = run_gpu(x, torch.bfloat16)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("name,dtype", [("heads_varlen", torch.bfloat16), ("varlen_mix", torch.bfloat16),
                                        ("varlen_mix", torch.float32)])
def test_packed_order_is_bitwise_neutral(name, dtype):
    """A packed batch given the workspace takes its sequences longest first;
    without it, in index order.  Only the assignment of sequences to
    workgroups differs, so outputs and final states are bitwise equal."""
    gdn = _gdn()
    dev = torch.device("cuda:0")
    x = oracle.add_gates(make_inputs(SMALL[name], seed=5, io_dtype=torch.float32))
    q, k, v = (x[n].to(dev, dtype) for n in ("q", "k", "v"))
    g, beta, cu = x["g"].to(dev), x["beta"].to(dev), x["cu_seqlens"].to(dev)
    s0 = None if x["initial_state"] is None else x["initial_state"].to(dev)
    _, T, H, K = q.shape
    HV, V, N = v.shape[2], v.shape[3], x["N"]
    shape = gdn.make_shape(1, T, H, HV, K, V, N, gdn.GDN_BF16 if dtype == torch.bfloat16 else gdn.GDN_F32)
    need = gdn.gdn_chunk_fwd_workspace_bytes(shape)
    assert need == ((4 * N + 255) // 256) * 256
    res = []
    for ws in (torch.empty(need, dtype=torch.uint8, device=dev), None):
        o = torch.full((1, T, HV, V), float("nan"), dtype=dtype, device=dev)
        f = torch.full((N, HV, K, V), float("nan"), device=dev)
        st = gdn.gdn_chunk_fwd(q, k, v, g, beta, x["scale"], x["use_l2norm"], s0, cu, o, f, shape, ws)
        torch.cuda.synchronize()
        assert st == 0, gdn.gdn_status_str(st)
        res.append((o, f))
    (o1, f1), (o2, f2) = res
    _say(f"[order] {name} {dtype}: N={N} lens={x['lens']}")
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def _many(n_seqs):
    """A packed batch of n_seqs short sequences (lengths 0..24, so that many
    share a chunk count and the order's ties are exercised)."""
    rng = np.random.default_rng(n_seqs)
    lens = tuple(int(x) for x in rng.integers(0, 25, n_seqs))
    return scaled(WORKLOADS["varlen"], f"many_{n_seqs}", H=2, HV=4, K=64, V=64, lengths=lens)


@pytest.mark.parametrize("n_seqs", [1024, 1025])
def test_packed_order_many_sequences(n_seqs):
    """The order at its largest batch (1024 sequences, ranked in one
    workgroup) and just past it (1025: index order): parity with the oracle,
    and bitwise equal with and without the workspace."""
    gdn = _gdn()
    dev = torch.device("cuda:0")
    x = oracle.add_gates(make_inputs(_many(n_seqs), seed=7, io_dtype=torch.float32))
    check_full(x, torch.bfloat16)
    q, k, v = (x[n].to(dev, torch.bfloat16) for n in ("q", "k", "v"))
    g, beta, cu = x["g"].to(dev), x["beta"].to(dev), x["cu_seqlens"].to(dev)
    s0 = None if x["initial_state"] is None else x["initial_state"].to(dev)
    _, T, H, K = q.shape
    HV, V, N = v.shape[2], v.shape[3], x["N"]
    shape = gdn.make_shape(1, T, H, HV, K, V, N, gdn.GDN_BF16)
    need = gdn.gdn_chunk_fwd_workspace_bytes(shape)
    assert need == (4096 if n_seqs == 1024 else 0)
    res = []
    for ws in (torch.empty(max(need, 1), dtype=torch.uint8, device=dev), None):
        o = torch.full((1, T, HV, V), float("nan"), dtype=torch.bfloat16, device=dev)
        f = torch.full((N, HV, K, V), float("nan"), device=dev)
        st = gdn.gdn_chunk_fwd(q, k, v, g, beta, x["scale"], x["use_l2norm"], s0, cu, o, f, shape, ws)
        torch.cuda.synchronize()
        assert st == 0, gdn.gdn_status_str(st)
        res.append((o, f))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def test_varlen_sequences_are_isolated():
    """NaN in one packed sequence stays inside that sequence."""
    x = oracle.add_gates(make_inputs(SMALL["varlen_mix"], seed=4, io_dtype=torch.float32))
    cu = x["cu_seqlens"].tolist()
    o1, f1 = run_gpu(x, torch.bfloat16)
    bad = 5   # the 200-token sequence
    x["v"][0, cu[bad] + 7] = float("nan")
    o2, f2 = run_gpu(x, torch.bfloat16)
    for n in range(len(cu) - 1):
        s = slice(cu[n], cu[n + 1])
        if n == bad:
            assert torch.isnan(o2[0, cu[bad] + 7:cu[bad + 1]]).any()
            assert torch.isnan(f2[n]).any()
        else:
            assert torch.equal(o1[0, s], o2[0, s]) and torch.equal(f1[n], f2[n])


def test_outputs_fully_written():
    x = oracle.add_gates(make_inputs(SMALL["varlen_mix"], seed=5, io_dtype=torch.float32))
    T, HV, V = x["v"].shape[1], x["v"].shape[2], x["v"].shape[3]
    out = torch.full((1, T, HV, V), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    fin = torch.full(x["initial_state"].shape, float("nan"), device="cuda:0")
    o, f = run_gpu(x, torch.bfloat16, out=out, final_state=fin)
    assert not torch.isnan(o).any() and not torch.isnan(f).any()


def test_wrapper_rejects_bad_caller_buffers():
    """Caller-given out / final_state buffers are written in place: a wrong
    shape, dtype or a non-contiguous view is refused before any launch."""
    x = oracle.add_gates(make_inputs(SMALL["varlen_mix"], seed=5, io_dtype=torch.float32))
    T, HV, V = x["v"].shape[1], x["v"].shape[2], x["v"].shape[3]
    N, K = x["initial_state"].shape[0], x["initial_state"].shape[2]
    dev = "cuda:0"
    bad_outs = [torch.empty((1, T, HV, V), dtype=torch.float32, device=dev),          # dtype
                torch.empty((1, T, HV, V + 1), dtype=torch.bfloat16, device=dev)[..., :V],   # strided view
                torch.empty((1, T + 1, HV, V), dtype=torch.bfloat16, device=dev)]          # shape
    for out in bad_outs:
        with pytest.raises(ValueError):
            run_gpu(x, torch.bfloat16, out=out)
    with pytest.raises(ValueError):
        run_gpu(x, torch.bfloat16, final_state=torch.empty((N, HV, V, K + 1), device=dev))


def test_empty_batch():
    w = scaled(WORKLOADS["varlen"], "empty", H=2, HV=4, lengths=(0, 0, 0))
    x = oracle.add_gates(make_inputs(w, seed=6, io_dtype=torch.float32))
    o, f = run_gpu(x, torch.bfloat16)
    assert o.numel() == 0
    assert torch.equal(f.cpu(), x["initial_state"])


# ---------------------------------------------------------------------------
# Full-size workloads: sampled units, same launch configuration as the bench.
# ---------------------------------------------------------------------------
FULL = {"gva": (WORKLOADS["gva"], 6), "varlen": (WORKLOADS["varlen"], 6),
        "long": (WORKLOADS["long"], 1), "wide_stable": (WORKLOADS["wide_stable"], 4)}


def _sample_units(x, count, seed=0):
    N, HV = x["N"], x["workload"].HV
    rng = np.random.default_rng(seed)
    units = {0, N * HV - 1}
    lens = x["lens"]
    units.add(int(np.argmax(lens)) * HV + HV // 2)
    while len(units) < count:
        units.add(int(rng.integers(0, N * HV)))
    return sorted(units)[:max(count, 2)]


def _full_size(name, dtype):
    w, count = FULL[name]
    _say(f"[parity-full] {name} {dtype}: generating on the GPU")
    x = oracle.add_gates(make_inputs(w, seed=0, device="cuda:0", io_dtype=dtype))
    o, fin = run_gpu(x, dtype)
    assert torch.isfinite(o).all() and torch.isfinite(fin).all()
    units = _sample_units(x, count)
    HV = w.HV
    G = HV // w.H
    cu = x["cu_seqlens"]
    starts = ([int(c) for c in cu.tolist()] if cu is not None else [n * w.T for n in range(x["N"] + 1)])
    for u in units:
        n, j = divmod(u, HV)
        t0, t1 = starts[n], starts[n + 1]
        jk = j // G

        def sl(t, head):
            return t.reshape(-1, *t.shape[2:])[t0:t1, head:head + 1].unsqueeze(0).cpu()
        s0 = None if x["initial_state"] is None else x["initial_state"][n:n + 1, j:j + 1].cpu()
        o_ref, f_ref = oracle.recurrent(sl(x["q"], jk), sl(x["k"], jk), sl(x["v"], j),
                                        sl(x["g"], j),
                                        sl(x["beta"], j), scale=x["scale"], use_l2norm=x["use_l2norm"],
                                        initial_state=s0, nthreads=8)
        og = o.reshape(-1, HV, w.V)[t0:t1, j].float().cpu().numpy()
        err = np.abs(og - o_ref[0, :, 0])
        eo = float(err.max()) if t1 > t0 else 0.0
        ef = float(np.abs(fin[n, j].cpu().numpy() - f_ref[0, 0]).max())
        _say(f"    unit n={n} j={j} len={t1 - t0}:")
        check_errors(eo, ef, o_ref, f_ref[0, 0], dtype)
        if t1 - t0 >= 8 * 4096:
            # the error must not grow late in the sequence: max error of every
            # 4096-token window; the last four windows against the first four
            win = err[:(t1 - t0) // 4096 * 4096].reshape(-1, 4096, err.shape[-1]).max(axis=(1, 2))
            _say("    per 4096-token window: " + " ".join(f"{e:.1e}" for e in win))
            assert win[-4:].max() <= 3 * win[:4].max(), "error grows late in the sequence"


@pytest.mark.parametrize("name", list(FULL))
def test_parity_full_size_sampled(name):
    _full_size(name, torch.bfloat16)


@pytest.mark.parametrize("name", list(FULL))
def test_parity_full_size_sampled_fp32(name):
    """The fp32 check mode (1e-4) at the full sizes, same sampled units."""
    _full_size(name, torch.float32)
