"""Host-side checks of bench.py (no GPU): the multi-GPU refusal, the byte and
flop accounting the roofline uses, and the traffic keying."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import DECODE_WORKLOADS, WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_prefill_bytes_and_flops_of_the_gva_workload():
    w = WORKLOADS["gva"]
    x = {"lens": [w.T] * w.B, "N": w.B, "initial_state": object()}
    T_tot = w.B * w.T
    # per token and value head: q, k (per key head, G = 2 value heads share them), v, o in bf16, g, beta fp32
    per_tok = (2 * w.H * w.K * 2 + 2 * w.HV * w.V * 2 + 8 * w.HV) / w.HV
    assert per_tok == 776
    states = 2 * w.B * w.HV * w.K * w.V * 4
    assert bench.path_bytes(w, x, 2) == T_tot * w.HV * 776 + states == 423624704
    # in-kernel gating reads a, b (bf16) and A_log, dt_bias instead of g, beta
    assert bench.path_bytes(w, x, 2, fused=True) == 423624704 - T_tot * w.HV * 4 + 8 * w.HV
    assert bench.path_flops(w, x) == T_tot * w.HV * (6 * 128 * 128 + 64 * (3 * 128 + 2 * 128))


def test_backward_bytes_and_flops_of_the_gva_workload():
    w = WORKLOADS["gva"]
    x = {"lens": [w.T] * w.B, "N": w.B, "initial_state": object()}
    T_tot = w.B * w.T
    state = w.B * w.HV * w.K * w.V * 4
    # reads q, k, v, do (bf16), g, beta, the initial state and dht; writes dq, dk, dv, dg, dbeta, dh0
    reads = 2 * T_tot * w.H * w.K * 2 + 2 * T_tot * w.HV * w.V * 2 + 8 * T_tot * w.HV + 2 * state
    writes = 2 * T_tot * w.H * w.K * 2 + T_tot * w.HV * w.V * 2 + 8 * T_tot * w.HV + state
    assert bench.bwd_path_bytes(w, x, 2) == reads + writes == 704643072
    # 16 K V + 6 C K + 5 C V + C^2 / 3 flops per token and value head, C = 64
    per_tok = 16 * 128 * 128 + 6 * 64 * 128 + 5 * 64 * 128 + 64 * 64 / 3
    assert bench.bwd_path_flops(w, x) == int(T_tot * w.HV * per_tok) == 185399421610


def test_decode_bytes():
    w = DECODE_WORKLOADS["decode"]
    assert bench.decode_bytes(w, 248, 2) == 1046412288
    wb = DECODE_WORKLOADS["decode_bf16pool"]
    assert bench.decode_bytes(wb, 248, 2) == 1046412288 - 248 * 32 * 128 * 128 * 4


def test_kernel_hash_ignores_comments(tmp_path):
    a = "int f(int x) {  // returns x\n  return x; /* plain */ }\n"
    b = "int f(int x) {\n  // another note\n  return x;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(a.replace("return x", "return -x"))
