#!/usr/bin/env python3
"""Throughput of the chunked gated delta rule forward pass on one MI355X
(``--path bwd``: its backward pass; a decode workload: the decode step).

One step = one full forward pass (every kernel of the path) over one batch of
seeded synthetic inputs already resident in HBM.  Default workload (the
headline): the wide large-batch prefill, B=16, T=16384, H=32 key heads, HV=64
value heads, K=V=128, bf16, no L2 norm, scale 1/sqrt(128), fp32 initial and
final state -- the largest configuration of the five, timed on its literal
inputs (which diverge; timing does not depend on the values).  After the
headline's timed region the other four configurations (tiny, GVA, packed
varlen, long) are timed the same way and reported under "configs".

Prints one JSON line: tokens/s, the roofline position of the path (timed live
with HIP events through the library's timing hook), and the fp64 oracle timed
on this host's cores on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "chunk GDN prefill tokens/s on 1 MI355X; % of bf16 MFMA / HBM roofline"

# HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled by a
# 1 GiB copy; see profiles/*_hbm_traffic.md), keyed by a hash of the measured
# kernel's source, the device headers and the compile flags.  Any change to them
# changes the hash, and the bench then reports traffic as null until it is
# measured again.
MEASURED_TRAFFIC = {
    # fused_ws_kernel (profiles/fused_ws_kernel_*_hbm_traffic.md, split_long_hbm_traffic.md):
    # wide FETCH 4,929,002.3 KiB x 2.000 + WRITE 4,259,873.5 KiB x 1.000; GVA 151,794.4 x 2 + 139,269.4;
    # varlen 627,216.9 x 2 + 630,164.0; long: the mean of its three fused launches per step
    # (925,869.2 x 2 + 16,384.0, 394,391.0 x 2 + 16,384.0 and the output pass's median)
    "4727c299a14c8c66": {"wide": 14456456905, "gva": 453471854, "varlen": 1929757539, "long": 2130635945},
    # recurrent_update_kernel: decode (fp32 pool) FETCH 257,459.5 x 2 + WRITE 510,374.0 KiB;
    # decode_bf16pool FETCH 130,489.5 x 2 + WRITE 256,178.2 KiB (counted under 1e133469e85525fe;
    # the headers changed since in declarations the decode kernel does not use, and its gfx950
    # assembly is identical)
    "7353cb8091568e35": {"decode": 1049900032, "decode_bf16pool": 529568973},
    # backward (GVA, varlen, wide): every kernel's FETCH x 2.000 + WRITE (profiles/backward_gva_hbm_traffic.md)
    "4d0f866784339036": {"gva:bwd_prep_kernel": 420070202, "gva:bwd_fwd_scan_kernel": 1199725144,
                         "gva:bwd_dh_scan_kernel": 1426231011, "gva:bwd_grads_kernel": 3359121488,
                         "gva:bwd_reduce_kernel": 671081344, "varlen:bwd_setup_kernel": 6047,
                         "varlen:bwd_prep_kernel": 2589382046, "varlen:bwd_fwd_scan_kernel": 5722425038,
                         "varlen:bwd_dh_scan_kernel": 7540025768, "varlen:bwd_grads_kernel": 12755039888,
                         "varlen:bwd_reduce_kernel": 2555238216, "wide:bwd_prep_kernel": 21515179463,
                         "wide:bwd_fwd_scan_kernel": 46239522806, "wide:bwd_dh_scan_kernel": 60475926204,
                         "wide:bwd_grads_kernel": 108938610336, "wide:bwd_reduce_kernel": 21474298897},
}
# Counter-based utilisation of the prefill kernel (profiles/fused_ws_kernel_wide_gva_sq_counters.md),
# keyed like MEASURED_TRAFFIC: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES over SIMD cycles, LDS busy and
# LDS bank-conflict stalls from SQ_LDS_IDX_ACTIVE and SQ_LDS_BANK_CONFLICT over cycles.
MEASURED_COUNTERS = {
    "4727c299a14c8c66": {"wide": {"mfma_busy": 0.450, "lds_busy": 0.677, "lds_bank_conflict": 0.124},
                         "gva": {"mfma_busy": 0.314, "lds_busy": 0.483, "lds_bank_conflict": 0.075}},
}
KERNEL_SOURCES = {
    "prefill": ["gated_deltanet_chunked_delta_amd/csrc/gdn_fused_ws.hip"],
    "decode": ["gated_deltanet_chunked_delta_amd/csrc/gdn_recurrent.hip"],
    "backward": ["gated_deltanet_chunked_delta_amd/csrc/gdn_backward.hip"],
}
DEVICE_HEADERS = ["gated_deltanet_chunked_delta_amd/csrc/gdn_device.h",
                  "gated_deltanet_chunked_delta_amd/csrc/gdn_internal.h"]


def _code_only(text):
    """Source text without comments and with whitespace collapsed, so that a
    change to comments alone keeps the hash."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_hash(kind):
    import hashlib
    from gated_deltanet_chunked_delta_amd import build as gbuild
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind] + DEVICE_HEADERS:
        h.update(_code_only(open(os.path.join(ROOT, f)).read()).encode())
    h.update(" ".join(gbuild.HIPCC_FLAGS).encode())
    return h.hexdigest()[:16]


def copy_calibration(mib, dev):
    """One plain device copy of known size, the reference kernel for the byte
    counters (run only when asked, after the timed region)."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
SETTLE_S = 0.1                 # untimed launches before the warmup steps (clock settling)
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}   # dense MFMA


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="wide")
    ap.add_argument("--configs", default="tiny,gva,varlen,long",
                    help="further forward workloads timed after the headline (comma list; empty: none)")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp32"])
    ap.add_argument("--cpu-units", type=int, default=0, help="oracle units for the CPU baseline (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gating", default="tensors", choices=["tensors", "fused", "separate"],
                    help="tensors: g and beta are inputs (computed once by the gating kernel before timing); "
                         "fused: the kernel computes them from A_log, dt_bias, a, b; separate: each step runs "
                         "the gating kernel, then the kernel with g and beta")
    ap.add_argument("--path", default="fwd", choices=["fwd", "bwd"],
                    help="fwd: the forward pass (prefill); bwd: the backward pass (gdn_chunk_bwd) of the "
                         "same workload, given the output and final-state gradients")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, run one plain device-to-device copy of this many MiB "
                         "(a reference kernel of known traffic for hardware byte counters)")
    return ap.parse_args()


def gate_bytes(rows, HV, eb, fused):
    """Gate inputs read by the chunk or decode kernel: g and beta (fp32) per
    row and value head, or with in-kernel gating a and b (eb bytes) per row and
    value head plus A_log and dt_bias per value head."""
    return rows * HV * 2 * eb + 8 * HV if fused else rows * HV * 8


def path_bytes(w, x, eb, fused=False):
    """Algorithmic HBM bytes of one forward pass: every input read once and
    every output written once (q, k per key head; v, the gates, o per value
    head; the initial and final states)."""
    T_tot = sum(x["lens"])
    N, H, HV, K, V = x["N"], w.H, w.HV, w.K, w.V
    s_in = N * HV * K * V * 4 if x["initial_state"] is not None else 0
    return (2 * T_tot * H * K * eb + T_tot * HV * V * eb + gate_bytes(T_tot, HV, eb, fused) + T_tot * HV * V * eb
            + s_in + N * HV * K * V * 4)


def path_flops(w, x):
    """Algorithmic flops of the method per forward pass: per token and value
    head 6KV (W.h, K^T.V_new, Q.h) + C(3K + 2V) (the causal intra-chunk
    products K.K^T, Q.K^T, the W recompute, U and P.V_new), C = 64."""
    T_tot = sum(x["lens"])
    return T_tot * w.HV * (6 * w.K * w.V + 64 * (3 * w.K + 2 * w.V))


def cpu_baseline(x, units_wanted):
    import numpy as np
    import oracle
    w = x["workload"]
    N, HV = x["N"], w.HV
    ncpu = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    U = units_wanted or min(N * HV, max(6 * ncpu, 16))
    units = np.unique(np.linspace(0, N * HV - 1, U).round().astype(np.int64))
    threads = int(min(ncpu, len(units)))
    cpu = lambda t: None if t is None else t.cpu()
    args = [cpu(x[n]) for n in ("q", "k", "v")]
    raw = [cpu(x[n]) for n in ("A_log", "dt_bias", "a", "b")]
    s0 = cpu(x["initial_state"])
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].cpu().numpy()
    t0 = time.perf_counter()
    oracle.recurrent_gated(*args, *raw, scale=x["scale"], use_l2norm=x["use_l2norm"], initial_state=s0,
                           cu_seqlens=cu, units=units, nthreads=threads)
    dt = time.perf_counter() - t0
    lens = x["lens"]
    unit_tokens = sum(lens[int(u) // HV] for u in units)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), model)
    except OSError:
        pass
    return {"value": unit_tokens / HV / dt, "unit": "tokens/s", "cores": threads, "nproc": os.cpu_count(),
            "cpu_model": model, "kind": "oracle",
            "sample": f"{len(units)} of {N * HV} (sequence, value head) units of the same inputs "
                      f"({unit_tokens} unit-tokens, fp64 gates and token recurrence, {dt:.2f} s wall)",
            "seconds": dt}


DECODE_METRIC = "fused recurrent GDN decode tokens/s on 1 MI355X (one token per sequence, pool-indexed state)"


def decode_bytes(w, n_valid, eb, fused=False):
    """Algorithmic HBM bytes of one decode step: each valid row reads q, k (per
    key head), v, its gates and its K x V state (fp32 or bf16), writes o and
    the state; padded rows write o; every row reads its slot index."""
    import torch
    N = w.N
    sb = 2 if w.pool_dtype == torch.bfloat16 else 4
    return (n_valid * (2 * w.H * w.K * eb + w.HV * w.V * eb + 2 * sb * w.HV * w.K * w.V)
            + gate_bytes(n_valid, w.HV, eb, fused) + N * w.HV * w.V * eb + 4 * N)


def run_decode(args):
    import torch
    import gated_deltanet_chunked_delta_amd as gdn
    from workloads import DECODE_WORKLOADS, make_decode_inputs

    w = DECODE_WORKLOADS[args.workload]
    dtype = torch.bfloat16 if args.dtype == "bf16" else torch.float32
    eb = 2 if args.dtype == "bf16" else 4
    dev = torch.device("cuda:0")
    x = make_decode_inputs(w, seed=0, device=dev, io_dtype=dtype)
    n_valid = int((x["idx"] >= 0).sum())
    gates = gdn.make_gates(x["A_log"], x["dt_bias"], x["a"], x["b"])
    gt = torch.empty((w.N, w.HV), dtype=torch.float32, device=dev)
    bt = torch.empty_like(gt)
    gdt = gdn.GDN_BF16 if eb == 2 else gdn.GDN_F32
    if args.gating == "tensors":
        x["g"], x["beta"] = gdn.fused_gdn_gating(x["A_log"], x["a"], x["b"], x["dt_bias"])
    shape = gdn.make_decode_shape(w.N, w.H, w.HV, w.K, w.V, w.pool_size,
                                  gdn.GDN_BF16 if eb == 2 else gdn.GDN_F32)
    out = torch.empty((w.N, w.HV, w.V), dtype=dtype, device=dev)
    pool = x["pool"]
    stream = torch.cuda.current_stream(dev).cuda_stream
    pool_cpu0 = pool.cpu() if not args.no_cpu_baseline else None

    spool = gdn.make_state_pool(pool, x["idx"]) if pool.dtype == torch.bfloat16 else None

    def step():
        if spool is not None:   # a bf16 pool: the pool entry point
            g, beta = x.get("g"), x.get("beta")
            if args.gating == "separate":
                st = gdn.gdn_gating(gates, w.N, w.HV, gdt, gt, bt, stream=stream)
                if st != 0:
                    raise gdn.GdnError(st)
                g, beta = gt, bt
            st = gdn.gdn_recurrent_update_pool(x["q"], x["k"], x["v"], g, beta,
                                               gates if args.gating == "fused" else None, x["scale"],
                                               x["use_l2norm"], spool, out, shape, stream=stream)
        elif args.gating == "fused":
            st = gdn.gdn_recurrent_update_gated(x["q"], x["k"], x["v"], gates, x["scale"], x["use_l2norm"],
                                                pool, x["idx"], out, shape, stream=stream)
        else:
            g, beta = x.get("g"), x.get("beta")
            if args.gating == "separate":
                st = gdn.gdn_gating(gates, w.N, w.HV, gdt, gt, bt, stream=stream)
                if st != 0:
                    raise gdn.GdnError(st)
                g, beta = gt, bt
            st = gdn.gdn_recurrent_update(x["q"], x["k"], x["v"], g, beta, x["scale"], x["use_l2norm"],
                                          pool, x["idx"], out, shape, stream=stream)
        if st != 0:
            raise gdn.GdnError(st)

    settle = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(10):
            step()
        settle += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    gdn.gdn_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = gdn.gdn_profile_read()
    gdn.gdn_profile_enable(False)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib, dev)

    ms = (t1 - t0) * 1e3 / args.steps
    kernels = {k: {"avg_us": 1e3 * t / n, "launches": n} for k, (t, n) in prof.items() if n}
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches"])
    dom_us = kernels[dom]["avg_us"]
    pb = decode_bytes(w, n_valid, eb, fused=args.gating == "fused")
    ach = pb / (dom_us * 1e-6) / 1e9
    khash = kernel_hash("decode")
    traffic = (MEASURED_TRAFFIC.get(khash, {}).get(w.name)
               if args.dtype == "bf16" and args.gating == "tensors" else None)
    res = {
        "metric": DECODE_METRIC, "value": round(n_valid / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_steps": settle, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: N={w.N} (valid {n_valid}) H={w.H} HV={w.HV} K={w.K} V={w.V} "
                               f"pool={w.pool_size} ({str(w.pool_dtype)[6:]}) l2norm={w.use_l2norm} "
                               f"gating={args.gating}",
                   "tokens": n_valid, "global_batch": w.N, "seq_len": 1, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": pb, "avg_launch_us": round(dom_us, 2),
                     "kernel_hash": khash},
        "kernels": {k: {kk: round(vv, 2) if isinstance(vv, float) else vv for kk, vv in v.items()}
                    for k, v in kernels.items()},
    }
    if not args.no_cpu_baseline:
        import oracle
        ncpu = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
        valid = (x["idx"] >= 0).cpu()
        sel = torch.nonzero(valid).flatten()
        cpu = lambda t: t.cpu()[sel].unsqueeze(1)
        s0 = pool_cpu0[x["idx"].cpu()[sel].long()]
        t2 = time.perf_counter()
        oracle.recurrent_gated(cpu(x["q"]), cpu(x["k"]), cpu(x["v"]), x["A_log"].cpu(), x["dt_bias"].cpu(),
                               cpu(x["a"]), cpu(x["b"]), scale=x["scale"], use_l2norm=x["use_l2norm"],
                               initial_state=s0, nthreads=ncpu)
        dt = time.perf_counter() - t2
        res["cpu_baseline"] = {"value": round(len(sel) / dt, 1), "unit": "tokens/s", "cores": ncpu,
                               "kind": "oracle",
                               "sample": f"the whole step: {len(sel)} rows x {w.HV} value heads, fp64 gates "
                                         f"and token recurrence from the initial pool ({dt:.3f} s wall)"}
    print(json.dumps(res), flush=True)


BWD_METRIC = "chunk GDN backward tokens/s on 1 MI355X (dq, dk, dv, dg, dbeta, dh0)"


def bwd_path_bytes(w, x, eb):
    """Algorithmic HBM bytes of one backward pass: every input read once (q, k
    per key head; v, do, g, beta per value head; the initial state and the
    final-state gradient) and every gradient written once (dq, dk per key head;
    dv, dg, dbeta per value head; dh0)."""
    T_tot = sum(x["lens"])
    N, H, HV, K, V = x["N"], w.H, w.HV, w.K, w.V
    state = N * HV * K * V * 4
    s_in = state if x["initial_state"] is not None else 0
    reads = 2 * T_tot * H * K * eb + 2 * T_tot * HV * V * eb + T_tot * HV * 8 + s_in + state
    writes = 2 * T_tot * H * K * eb + T_tot * HV * V * eb + T_tot * HV * 8 + state
    return reads + writes


def bwd_path_flops(w, x):
    """Algorithmic flops of one backward pass: the products of the chain rule
    through the chunked form, per chunk of C = 64 rows with the triangular
    masks counted (2 flops per multiply-add).  Per token and value head: eight
    C x K x V products per chunk (the forward rescan's Kh h and Kh^T F, then
    Kh dh', Qh^T dO, Kh^T dB, dO h^T, dB h^T, Vn dh'^T) give 16 K V; six
    half-masked C x C x K products (K K^T, Q K^T, dSqk Kh, dSqk^T Qh, Ad Kh,
    Ad^T Kh) give 6 C K; five half-masked C x C x V products (Tm B, Pm^T dO,
    Tm^T dVn, dO Vn^T, dB Vn^T) give 5 C V; the triangular inverse C^2 / 3."""
    C = 64
    per_tok = 16 * w.K * w.V + 6 * C * w.K + 5 * C * w.V + C * C / 3
    return int(sum(x["lens"]) * w.HV * per_tok)


def bwd_cpu_baseline(x, groups=2):
    """The fp64 backward oracle (numpy, token by token) on `groups` (sequence,
    key head) groups of the same inputs, with all value heads of each group."""
    import numpy as np
    from oracle.backward import backward
    w = x["workload"]
    G = w.HV // w.H
    N = x["N"]
    picks = [(int(n), int(h)) for n, h in zip(np.linspace(0, N - 1, groups).round(),
                                              np.linspace(0, w.H - 1, groups).round())]
    toks = 0
    t0 = time.perf_counter()
    for n, jk in picks:
        sl = slice(jk * G, (jk + 1) * G)
        c = lambda t: t[n:n + 1].cpu()
        s0 = None if x["initial_state"] is None else x["initial_state"][n:n + 1, sl].cpu()
        backward(c(x["q"])[:, :, jk:jk + 1], c(x["k"])[:, :, jk:jk + 1], c(x["v"])[:, :, sl],
                 c(x["g"])[:, :, sl], c(x["beta"])[:, :, sl], c(x["do"])[:, :, sl], dht=x["dht"][n:n + 1, sl].cpu(),
                 scale=x["scale"], use_l2norm=x["use_l2norm"], initial_state=s0)
        toks += x["lens"][n] * G
    dt = time.perf_counter() - t0
    return {"value": round(toks / w.HV / dt, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(picks)} (sequence, key head) groups x {G} value heads of the same inputs "
                      f"({toks} unit-tokens, fp64 token-level reverse mode in numpy, {dt:.2f} s wall)"}


def run_backward(args):
    import torch
    import gated_deltanet_chunked_delta_amd as gdn
    from workloads import WORKLOADS, make_grad_inputs, make_inputs

    w = WORKLOADS[args.workload]
    dtype = torch.bfloat16 if args.dtype == "bf16" else torch.float32
    eb = 2 if args.dtype == "bf16" else 4
    dev = torch.device("cuda:0")
    x = make_inputs(w, seed=0, device=dev, io_dtype=dtype)
    x["g"], x["beta"] = gdn.fused_gdn_gating(x["A_log"], x["a"], x["b"], x["dt_bias"])
    x = make_grad_inputs(x, seed=100)
    B, T = x["q"].shape[0], x["q"].shape[1]
    N = x["N"]
    shape = gdn.make_shape(B, T, w.H, w.HV, w.K, w.V, N, gdn.GDN_BF16 if eb == 2 else gdn.GDN_F32)
    ws = torch.empty(gdn.gdn_chunk_bwd_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
    dg = torch.empty((B, T, w.HV), dtype=torch.float32, device=dev)
    dbeta = torch.empty_like(dg)
    dh0 = torch.empty((N, w.HV, w.K, w.V), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def step():
        st = gdn.gdn_chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], x["dht"], x["scale"],
                               x["use_l2norm"], x["initial_state"], x["cu_seqlens"], dq, dk, dv, dg, dbeta, dh0,
                               shape, ws, stream=stream)
        if st != 0:
            raise gdn.GdnError(st)

    settle = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < SETTLE_S:
        step()
        settle += 1
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    gdn.gdn_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = gdn.gdn_profile_read()
    gdn.gdn_profile_enable(False)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib, dev)

    tokens = sum(x["lens"])
    ms = (t1 - t0) * 1e3 / args.steps
    pb = bwd_path_bytes(w, x, eb)
    kernels = {k: {"avg_us": 1e3 * t / n, "launches": n} for k, (t, n) in prof.items() if n}
    per_step = lambda k: kernels[k]["avg_us"] * kernels[k]["launches"] / args.steps
    dom = max(kernels, key=per_step)
    path_us = sum(per_step(k) for k in kernels)
    # five kernels share the path: the path's algorithmic bytes over the sum of
    # their times per step (the dominant kernel's share of that time is given)
    ach = pb / (path_us * 1e-6) / 1e9
    flops = bwd_path_flops(w, x)
    tflops = flops / (path_us * 1e-6) / 1e12
    khash = kernel_hash("backward")
    traffic = MEASURED_TRAFFIC.get(khash, {}).get(w.name + ":" + dom)
    res = {
        "metric": BWD_METRIC, "value": round(tokens / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_steps": settle, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name} backward: B={B} T={T} N={N} H={w.H} HV={w.HV} K={w.K} V={w.V} "
                               f"l2norm={w.use_l2norm} initial_state={w.init} dht=yes",
                   "tokens": tokens, "global_batch": N, "seq_len": T if N == B else None,
                   "parallelism": "single GPU"},
        # every product runs in fp32 on the matrix cores and the pass does ~260
        # flops per algorithmic byte, far above the fp32 ridge (157.3 TFLOP/s
        # over 8 TB/s = 20 flop/B): the bound is fp32 MFMA, the HBM side is given
        "roofline": {"bound": "mfma", "dtype": "fp32", "scope": "path", "kernel": dom,
                     "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS["fp32"], "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_PEAK_TFLOPS["fp32"], 4), "traffic": traffic,
                     "traffic_scope": "dominant kernel, bytes per launch", "kernel_hash": khash,
                     "algorithmic_flops_per_step": flops, "algorithmic_bytes_per_step": pb,
                     "hbm_frac": round(ach / HBM_PEAK_GBS, 4), "kernel_us_per_step": round(path_us, 2),
                     "dominant_kernel_share": round(per_step(dom) / path_us, 3)},
        "kernels": {k: {kk: round(vv, 2) if isinstance(vv, float) else vv for kk, vv in v.items()}
                    for k, v in kernels.items()},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = bwd_cpu_baseline(x)
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    from workloads import DECODE_WORKLOADS
    if args.workload in DECODE_WORKLOADS:
        run_decode(args)
        return
    if args.path == "bwd":
        run_backward(args)
        return

    res = run_forward(args, args.workload, args.steps, args.warmup, headline=True)
    if args.configs and args.dtype == "bf16" and args.gating == "tensors":
        # the other configurations, measured after the headline's timed region
        res["configs"] = {}
        for name in [c for c in args.configs.split(",") if c and c != args.workload]:
            r = run_forward(args, name, max(5, args.steps // 2), max(2, args.warmup // 2), headline=False)
            res["configs"][name] = r
    print(json.dumps(res), flush=True)


def run_forward(args, name, steps, warmup, headline):
    """Times `steps` forward passes of workload `name` (after the clocks settle
    and `warmup` untimed passes) and returns the bench record (headline) or a
    short summary (the other configurations)."""
    import torch
    import gated_deltanet_chunked_delta_amd as gdn
    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[name]
    dtype = torch.bfloat16 if args.dtype == "bf16" else torch.float32
    eb = 2 if args.dtype == "bf16" else 4
    dev = torch.device("cuda:0")
    x = make_inputs(w, seed=0, device=dev, io_dtype=dtype)
    B, T = x["q"].shape[0], x["q"].shape[1]
    N = x["N"]
    gates = gdn.make_gates(x["A_log"], x["dt_bias"], x["a"], x["b"])
    gt = torch.empty((B, T, w.HV), dtype=torch.float32, device=dev)
    bt = torch.empty_like(gt)
    gdt = gdn.GDN_BF16 if eb == 2 else gdn.GDN_F32
    if args.gating == "tensors":
        x["g"], x["beta"] = gdn.fused_gdn_gating(x["A_log"], x["a"], x["b"], x["dt_bias"])
    shape = gdn.make_shape(B, T, w.H, w.HV, w.K, w.V, N, gdn.GDN_BF16 if eb == 2 else gdn.GDN_F32)
    need = gdn.gdn_chunk_fwd_workspace_bytes(shape)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    out = torch.empty((B, T, w.HV, w.V), dtype=dtype, device=dev)
    fin = torch.empty((N, w.HV, w.K, w.V), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def step():
        if args.gating == "fused":
            st = gdn.gdn_chunk_fwd_gated(x["q"], x["k"], x["v"], gates, x["scale"], x["use_l2norm"],
                                         x["initial_state"], x["cu_seqlens"], out, fin, shape, ws, stream=stream)
        else:
            g, beta = x.get("g"), x.get("beta")
            if args.gating == "separate":
                st = gdn.gdn_gating(gates, B * T, w.HV, gdt, gt, bt, stream=stream)
                if st != 0:
                    raise gdn.GdnError(st)
                g, beta = gt, bt
            st = gdn.gdn_chunk_fwd(x["q"], x["k"], x["v"], g, beta, x["scale"], x["use_l2norm"],
                                   x["initial_state"], x["cu_seqlens"], out, fin, shape, ws, stream=stream)
        if st != 0:
            raise gdn.GdnError(st)

    # Settle: the clocks of a freshly busy GPU take ~100 launches of this size
    # to reach their steady state (kernel times dip and recover meanwhile), so
    # untimed launches run for at least SETTLE_S seconds before the W warmup steps.
    settle = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(10):
            step()
        settle += 10
        torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    gdn.gdn_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = gdn.gdn_profile_read()
    gdn.gdn_profile_enable(False)

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib, dev)

    tokens = sum(x["lens"])
    ms = (t1 - t0) * 1e3 / steps
    value = tokens / (ms / 1e3)
    pb = path_bytes(w, x, eb, fused=args.gating == "fused")
    kernels = {k: {"avg_us": 1e3 * t / n, "launches": n} for k, (t, n) in prof.items() if n}
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches"])
    dom_us = kernels[dom]["avg_us"]
    per_step = lambda k: kernels[k]["avg_us"] * kernels[k]["launches"] / steps
    path_us = sum(per_step(k) for k in kernels)
    # the path's algorithmic bytes over the time of every kernel of a step (the
    # fused kernel alone for most sizes; a split long sequence adds its setup,
    # combine and final-copy kernels and launches the fused kernel three times)
    ach = pb / (path_us * 1e-6) / 1e9
    khash = kernel_hash("prefill")
    traffic = (MEASURED_TRAFFIC.get(khash, {}).get(w.name)
               if args.dtype == "bf16" and args.gating == "tensors" else None)
    roof = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": pb, "avg_launch_us": round(dom_us, 2),
            "launches_per_step": round(kernels[dom]["launches"] / steps, 2), "kernel_hash": khash,
            "scope": "path" if len(kernels) > 1 else "kernel",
            "counters": (MEASURED_COUNTERS.get(khash, {}).get(w.name)
                         if args.dtype == "bf16" and args.gating == "tensors" else None)}
    flops = path_flops(w, x)
    path = {"algorithmic_bytes": pb, "algorithmic_flops": flops, "kernel_us": round(path_us, 2),
            "hbm_frac": round(pb / (path_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac": round(flops / (path_us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS[args.dtype], 4),
            "roofline_tokens_per_s": round(tokens / max(pb / (HBM_PEAK_GBS * 1e9),
                                                         flops / (MFMA_PEAK_TFLOPS[args.dtype] * 1e12)))}
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "settle_steps": settle, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: B={B} T={T} N={N} H={w.H} HV={w.HV} K={w.K} V={w.V} "
                               f"l2norm={w.use_l2norm} initial_state={w.init} gating={args.gating}",
                   "tokens": tokens, "global_batch": N, "seq_len": T if N == B else None,
                   "parallelism": "single GPU"},
        "roofline": roof, "path": path,
        "kernels": {k: {kk: round(vv, 2) if isinstance(vv, float) else vv for kk, vv in v.items()}
                    for k, v in kernels.items()},
    }
    if w.name == "wide":
        # the literal wide inputs diverge (no L2 norm, |k|^2 ~ K): the share of
        # finite outputs, for the record; timing does not depend on the values
        res["finite_output_fraction"] = round(float(torch.isfinite(out).float().mean()), 6)
    if not headline:
        return {"tokens": tokens, "tokens_per_s": round(value, 1), "ms_per_step": round(ms, 4),
                "steps": steps, "hbm_frac": path["hbm_frac"], "mfma_frac": path["mfma_frac"],
                "kernel_us": path["kernel_us"], "traffic": traffic,
                "workload": res["config"]["workload"], "kernels": res["kernels"]}
    if not args.no_cpu_baseline:
        cb = cpu_baseline(x, args.cpu_units)
        cb.pop("seconds")
        cb["value"] = round(cb["value"], 1)
        res["cpu_baseline"] = cb
    return res


if __name__ == "__main__":
    main()
