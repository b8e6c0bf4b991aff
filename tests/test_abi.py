"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/gdn.h declares, and
reject bad arguments on the host before anything is enqueued (the argument
pointers here are never dereferenced: every call below fails a check first).
"""
import ctypes
import os
import re

import pytest

import gated_deltanet_chunked_delta_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20   # a non-null address that is never touched


def declared_functions():
    text = open(os.path.join(ROOT, "include", "gdn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = gdn.load_library()
    names = declared_functions()
    assert names == sorted(gdn.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name


def test_header_compiles_as_c():
    import subprocess
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        open(src, "w").write('#include "gdn.h"\nint main(void){gdn_shape s={0};(void)s;return 0;}\n')
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), "-c", src,
                        "-o", os.path.join(d, "t.o")], check=True)


def _call(shape, ws=FAKE, ws_bytes=1 << 40, cu=None, ptrs=FAKE):
    lib = gdn.load_library()
    P = ctypes.c_void_p
    return lib.gdn_chunk_fwd(P(ptrs), P(ptrs), P(ptrs), P(ptrs), P(ptrs), 1.0, 1, None,
                             None if cu is None else P(cu), P(ptrs), None,
                             None if shape is None else ctypes.byref(shape), P(ws) if ws else None,
                             ws_bytes, None)


def test_workspace_size_and_bad_shapes():
    s1 = gdn.make_shape(4, 4096, 16, 32, 128, 128, 4, gdn.GDN_BF16)
    s2 = gdn.make_shape(4, 4096, 16, 32, 128, 128, 4, gdn.GDN_F32)
    b1, b2 = gdn.gdn_chunk_fwd_workspace_bytes(s1), gdn.gdn_chunk_fwd_workspace_bytes(s2)
    assert 0 <= b1 <= b2
    assert b1 == b2 == 0                      # 256 workgroups: not split
    # one long sequence (64 workgroups): split into 8 segments; the workspace holds
    # their start states, end states and transfer maps and the identity maps
    # (fp32), independent of T
    b3 = gdn.gdn_chunk_fwd_workspace_bytes(gdn.make_shape(1, 131072, 16, 32, 128, 128, 1, gdn.GDN_BF16))
    b4 = gdn.gdn_chunk_fwd_workspace_bytes(gdn.make_shape(1, 131072, 16, 32, 128, 128, 1, gdn.GDN_F32))
    b5 = gdn.gdn_chunk_fwd_workspace_bytes(gdn.make_shape(1, 4096, 16, 32, 128, 128, 1, gdn.GDN_BF16))
    states = 4 * 8 * 32 * 128 * (2 * 128 + 128) + 4 * 32 * 128 * 128
    assert states <= b3 < states + (1 << 20) and b4 >= b3 and b5 == b3
    assert gdn.gdn_chunk_fwd_workspace_bytes(gdn.make_shape(1, 1024, 16, 32, 128, 128, 1, 0)) == 0   # short
    # a packed batch: one int32 per sequence for the longest-first order, in
    # 256-byte granules, for 2..1024 sequences; none for one or for more
    assert gdn.gdn_chunk_fwd_workspace_bytes(gdn.make_shape(1, 1, 16, 32, 128, 128, 4, 0)) == 256
    assert gdn.gdn_chunk_fwd_workspace_bytes(gdn.make_shape(1, 5000, 16, 32, 128, 128, 64, 0)) == 256
    assert gdn.gdn_chunk_fwd_workspace_bytes(gdn.make_shape(1, 5000, 16, 32, 128, 128, 65, 0)) == 512
    assert gdn.gdn_chunk_fwd_workspace_bytes(gdn.make_shape(1, 5000, 2, 4, 64, 64, 1024, 1)) == 4096
    assert gdn.gdn_chunk_fwd_workspace_bytes(gdn.make_shape(1, 5000, 2, 4, 64, 64, 1025, 0)) == 0
    assert gdn.gdn_chunk_fwd_workspace_bytes(gdn.make_shape(1, 5000, 2, 4, 64, 64, 0, 0)) == 0
    assert gdn.gdn_chunk_fwd_workspace_bytes(gdn.make_shape(4, 4096, 16, 32, 96, 128, 4, 0)) == 0
    assert gdn.gdn_chunk_fwd_workspace_bytes(gdn.make_shape(4, 4096, 3, 32, 128, 128, 4, 0)) == 0
    assert gdn.gdn_chunk_fwd_workspace_bytes(gdn.make_shape(4, 4096, 16, 32, 128, 128, 4, 7)) == 0


@pytest.mark.parametrize("shape,cu,want", [
    (None, None, -1),                                           # no shape
    (gdn.make_shape(4, 64, 2, 4, 128, 128, 3, 0), None, -2),    # N != B without cu_seqlens
    (gdn.make_shape(2, 64, 2, 4, 128, 128, 2, 0), FAKE, -2),    # B != 1 with cu_seqlens
    (gdn.make_shape(1, -1, 2, 4, 128, 128, 1, 0), None, -2),    # negative T
    (gdn.make_shape(1, 64, 2, 4, 128, 128, 1, 5), None, -3),    # unknown dtype
    (gdn.make_shape(1, 64, 2, 4, 96, 128, 1, 0), None, -4),     # K not supported
    (gdn.make_shape(1, 64, 2, 4, 128, 32, 1, 0), None, -4),     # V not supported
    (gdn.make_shape(1, 64, 3, 4, 128, 128, 1, 0), None, -4),    # HV % H != 0
])
def test_argument_errors(shape, cu, want):
    assert _call(shape, cu=cu) == want


def test_null_tensor_errors():
    s = gdn.make_shape(1, 64, 2, 4, 128, 128, 1, 0)
    assert _call(s, ptrs=0) == -1


@pytest.mark.parametrize("arg,offset", [("q", 8), ("k", 2), ("v", 4), ("out", 8), ("initial_state", 4),
                                         ("final_state", 12), ("g", 2), ("beta", 1), ("cu_seqlens", 2)])
def test_forward_misaligned_pointers(arg, offset):
    """q, k, v, out and the states need 16-byte alignment, g, beta and
    cu_seqlens 4-byte: anything less is GDN_ERR_ALIGN, found on the host."""
    lib = gdn.load_library()
    P = ctypes.c_void_p
    ptr = {n: FAKE for n in ("q", "k", "v", "g", "beta", "initial_state", "out", "final_state")}
    ptr["cu_seqlens"] = None
    ptr[arg] = FAKE + offset
    s = gdn.make_shape(1, 64, 2, 4, 128, 128, 1, 0)
    args = [P(ptr[n]) if ptr[n] else None for n in ("q", "k", "v", "g", "beta")]
    st = lib.gdn_chunk_fwd(*args, 1.0, 1, P(ptr["initial_state"]),
                           None if ptr["cu_seqlens"] is None else P(ptr["cu_seqlens"]),
                           P(ptr["out"]), P(ptr["final_state"]), ctypes.byref(s), None, 0, None)
    assert st == -7


def test_noalloc_refuses_on_the_host():
    """gdn_chunk_fwd_noalloc checks like gdn_chunk_fwd on the host, and every
    split the library plans fits in its static scratch."""
    lib = gdn.load_library()
    P = ctypes.c_void_p
    call = lambda s, ptrs=FAKE: lib.gdn_chunk_fwd_noalloc(P(ptrs), P(ptrs), P(ptrs), P(ptrs), P(ptrs), 1.0, 1,
                                                          None, None, P(ptrs), None,
                                                          None if s is None else ctypes.byref(s), None)
    assert call(None) == -1
    assert call(gdn.make_shape(1, 64, 2, 4, 96, 128, 1, 0)) == -4
    assert gdn.GDN_ERR_SCRATCH == -8
    # every split the library plans fits in the static scratch (the workspace
    # grows with heads and segments, not with T)
    need = max(gdn.gdn_chunk_fwd_workspace_bytes(gdn.make_shape(B, T, 1, HV, K, V, B, dt))
               for K in (64, 128) for V in (64, 128) for B in (1, 2, 4, 16, 64) for HV in (1, 2, 8, 32, 64)
               for T in (2048, 5000, 131072) for dt in (0, 1))
    assert 0 < need <= gdn.GDN_STATIC_SCRATCH_BYTES
    # the constant of the header and of the binding agree
    hdr = open(os.path.join(ROOT, "include", "gdn.h")).read()
    assert "#define GDN_STATIC_SCRATCH_BYTES ((size_t)64 << 20)" in hdr
    assert gdn.GDN_STATIC_SCRATCH_BYTES == 64 << 20


def test_status_strings():
    for st in range(-8, 1):
        assert gdn.gdn_status_str(st).startswith("GDN_")
    assert gdn.gdn_status_str(-99) == "unknown gdn_status"


def test_python_wrapper_rejects_cpu_tensors_and_bad_shapes():
    import torch
    q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    v = torch.zeros(1, 8, 4, 64, dtype=torch.bfloat16)
    g = torch.zeros(1, 8, 4)
    with pytest.raises(ValueError):   # CPU tensors: there is no CPU path
        gdn.chunk_gated_delta_rule(q, q, v, g, g)
    with pytest.raises(ValueError):   # beta with H heads instead of HV
        gdn.chunk_gated_delta_rule(q, q, v, g, torch.zeros(1, 8, 2))


def _dcall(shape, ptrs=FAKE):
    lib = gdn.load_library()
    P = ctypes.c_void_p
    return lib.gdn_recurrent_update(P(ptrs), P(ptrs), P(ptrs), P(ptrs), P(ptrs), 1.0, 1, P(ptrs), P(ptrs),
                                    P(ptrs), None if shape is None else ctypes.byref(shape), None)


@pytest.mark.parametrize("shape,want", [
    (None, -1),                                                  # no shape
    (gdn.make_decode_shape(-1, 2, 4, 128, 128, 8, 0), -2),       # negative N
    (gdn.make_decode_shape(4, 2, 4, 128, 128, 0, 0), -2),        # empty pool with rows
    (gdn.make_decode_shape(4, 2, 4, 128, 128, 8, 9), -3),        # unknown dtype
    (gdn.make_decode_shape(4, 2, 4, 96, 128, 8, 0), -4),         # K not supported
    (gdn.make_decode_shape(4, 3, 4, 128, 128, 8, 0), -4),        # HV % H != 0
])
def test_decode_argument_errors(shape, want):
    assert _dcall(shape) == want


def _gates(A=FAKE, dt=FAKE, a=FAKE, b=FAKE):
    return gdn.gdn_gates(A, dt, a, b)


@pytest.mark.parametrize("gates,HV,dtype,want", [
    (None, 4, 0, -1),                        # no gates struct
    (dict(a=0), 4, 0, -1),                   # a missing
    (dict(A=0), 4, 0, -1),                   # A_log missing
    (dict(b=FAKE + 2), 4, 0, -7),            # b not 4-byte aligned
    ({}, 3, 0, -4),                          # bf16 gate inputs with odd HV
    ({}, 3, 9, -3),                          # unknown dtype
])
def test_prefill_gated_argument_errors(gates, HV, dtype, want):
    lib = gdn.load_library()
    P = ctypes.c_void_p
    shape = gdn.make_shape(2, 64, 1, HV, 128, 128, 2, dtype)
    gs = None if gates is None else ctypes.byref(_gates(**gates))
    assert lib.gdn_chunk_fwd_gated(P(FAKE), P(FAKE), P(FAKE), gs, 1.0, 1, None, None, P(FAKE), P(FAKE),
                                   ctypes.byref(shape), None, 0, None) == want


def test_gated_odd_hv_fp32_and_empty_are_accepted_on_the_host():
    # fp32 gate inputs have no word-sharing restriction; with no tokens and no
    # sequences nothing is launched, so FAKE pointers are never touched
    lib = gdn.load_library()
    P = ctypes.c_void_p
    shape = gdn.make_shape(0, 0, 1, 3, 128, 128, 0, 1)
    assert lib.gdn_chunk_fwd_gated(P(FAKE), P(FAKE), P(FAKE), ctypes.byref(_gates()), 1.0, 1, None, None,
                                   P(FAKE), None, ctypes.byref(shape), None, 0, None) == 0


@pytest.mark.parametrize("gates,want", [(None, -1), (dict(dt=0), -1), (dict(a=FAKE + 1), -7)])
def test_decode_gated_argument_errors(gates, want):
    lib = gdn.load_library()
    P = ctypes.c_void_p
    shape = gdn.make_decode_shape(4, 2, 4, 128, 128, 8, 0)
    gs = None if gates is None else ctypes.byref(_gates(**gates))
    assert lib.gdn_recurrent_update_gated(P(FAKE), P(FAKE), P(FAKE), gs, 1.0, 1, P(FAKE), P(FAKE), P(FAKE),
                                          ctypes.byref(shape), None) == want


@pytest.mark.parametrize("rows,HV,dtype,gates,want", [
    (-1, 4, 0, {}, -2), (4, 0, 0, {}, -2), (1 << 61, 4, 0, {}, -2), (4, 4, 5, {}, -3),
    (4, 4, 0, None, -1), (4, 4, 0, dict(b=0), -1), (4, 4, 0, dict(a=FAKE + 2), -7),
    (0, 4, 0, None, 0),                       # nothing to compute
])
def test_gating_argument_errors(rows, HV, dtype, gates, want):
    lib = gdn.load_library()
    P = ctypes.c_void_p
    gs = None if gates is None else ctypes.byref(_gates(**gates))
    assert lib.gdn_gating(gs, rows, HV, dtype, P(FAKE), P(FAKE), None) == want


@pytest.mark.parametrize("rows,HV,dtype,gates,null,ws,want", [
    (-1, 4, 0, {}, None, 1, -2), (4, 0, 0, {}, None, 1, -2), (4, 4, 5, {}, None, 1, -3),
    (4, 4, 0, None, None, 1, -1), (4, 4, 0, dict(dt=0), None, 1, -1),
    (4, 4, 0, {}, "dA_log", 1, -1), (4, 4, 0, {}, "dg", 1, -1), (4, 4, 0, {}, "db", 1, -1),
    (4, 4, 0, dict(a=FAKE + 2), None, 1, -7),
    (4, 4, 0, {}, None, 0, -5),                                  # workspace missing
    (4, 4, 0, {}, None, 2, -5),                                  # workspace misaligned
    (4, 4, 0, {}, None, 3, -5),                                  # workspace too small
])
def test_gating_bwd_argument_errors(rows, HV, dtype, gates, null, ws, want):
    lib = gdn.load_library()
    P = ctypes.c_void_p
    gs = None if gates is None else ctypes.byref(_gates(**gates))
    ptr = {n: (None if n == null else P(FAKE)) for n in ("dg", "dbeta", "da", "db", "dA_log", "ddt_bias")}
    need = gdn.gdn_gating_bwd_workspace_bytes(max(rows, 0), max(HV, 1))
    wsp, wsb = {0: (None, 0), 1: (P(FAKE), need), 2: (P(FAKE + 4), need), 3: (P(FAKE), need - 4)}[ws]
    assert lib.gdn_gating_bwd(gs, rows, HV, dtype, ptr["dg"], ptr["dbeta"], ptr["da"], ptr["db"], ptr["dA_log"],
                              ptr["ddt_bias"], wsp, wsb, None) == want


def test_gating_bwd_workspace_size():
    # two floats per head and 64-row block
    assert gdn.gdn_gating_bwd_workspace_bytes(1000, 32) == 2 * 16 * 32 * 4
    assert gdn.gdn_gating_bwd_workspace_bytes(64, 3) == 2 * 1 * 3 * 4
    assert gdn.gdn_gating_bwd_workspace_bytes(0, 32) == 0
    assert gdn.gdn_gating_bwd_workspace_bytes(-1, 32) == 0 and gdn.gdn_gating_bwd_workspace_bytes(8, 0) == 0


def test_gating_wrappers_reject_cpu_tensors_and_mixed_gates():
    import torch
    a = torch.zeros(3, 4, dtype=torch.bfloat16)
    A = torch.zeros(4)
    with pytest.raises(ValueError):
        gdn.fused_gdn_gating(A, a, a, A)
    q = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16)
    v = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    g = torch.zeros(1, 8, 2)
    with pytest.raises(ValueError):   # g and raw gates together
        gdn.chunk_gated_delta_rule(q, q, v, g, g, A_log=torch.zeros(2))


def _pool(data=FAKE, idx=FAKE, P=8, dtype=0, read=1):
    return gdn.gdn_state_pool(data, idx, P, dtype, read)


@pytest.mark.parametrize("pool,want", [
    (None, -1),                                  # no pool struct
    (dict(data=0), -1), (dict(idx=0), -1),       # pool without data / indices
    (dict(dtype=7), -3),                         # unknown pool dtype
    (dict(P=0), -2),                             # empty pool with sequences
    (dict(data=FAKE + 2, dtype=0), -7),          # a bf16 pool needs 8-byte alignment
    (dict(data=FAKE + 8, dtype=1), -7),          # an fp32 pool needs 16-byte alignment
])
def test_prefill_pool_argument_errors(pool, want):
    lib = gdn.load_library()
    P = ctypes.c_void_p
    shape = gdn.make_shape(2, 64, 1, 2, 128, 128, 2, 0)
    pl = None if pool is None else ctypes.byref(_pool(**pool))
    assert lib.gdn_chunk_fwd_pool(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, 1.0, 1, pl, None, P(FAKE),
                                  ctypes.byref(shape), None, 0, None) == want


@pytest.mark.parametrize("pool,pool_size,want", [
    (None, 8, -1), (dict(data=FAKE + 8, dtype=1), 8, -7), (dict(P=8), 9, -2), (dict(dtype=3), 8, -3),
])
def test_decode_pool_argument_errors(pool, pool_size, want):
    lib = gdn.load_library()
    P = ctypes.c_void_p
    shape = gdn.make_decode_shape(4, 2, 4, 128, 128, pool_size, 0)
    pl = None if pool is None else ctypes.byref(_pool(**pool))
    assert lib.gdn_recurrent_update_pool(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, 1.0, 1, pl, P(FAKE),
                                         ctypes.byref(shape), None) == want


def test_decode_misaligned_pool():
    lib = gdn.load_library()
    P = ctypes.c_void_p
    shape = gdn.make_decode_shape(4, 2, 4, 128, 128, 8, 0)
    assert lib.gdn_recurrent_update(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 1.0, 1, P(FAKE + 4), P(FAKE),
                                    P(FAKE), ctypes.byref(shape), None) == -7


def test_decode_null_and_empty():
    assert _dcall(gdn.make_decode_shape(4, 2, 4, 128, 128, 8, 0), ptrs=0) == -1
    # no rows: nothing to read or launch, NULL buffers allowed
    assert _dcall(gdn.make_decode_shape(0, 2, 4, 128, 128, 0, 0), ptrs=0) == 0


def test_decode_wrapper_rejects_cpu_tensors_and_bad_shapes():
    import torch
    q = torch.zeros(3, 2, 64, dtype=torch.bfloat16)
    v = torch.zeros(3, 4, 64, dtype=torch.bfloat16)
    g = torch.zeros(3, 4)
    pool = torch.zeros(5, 4, 64, 64)
    idx = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError):   # CPU tensors: there is no CPU path
        gdn.fused_recurrent_gated_delta_rule_update(q, q, v, g, g, pool, idx)
    with pytest.raises(ValueError):   # pool with the wrong head count
        gdn.fused_recurrent_gated_delta_rule_update(q, q, v, g, g, torch.zeros(5, 2, 64, 64), idx)
    with pytest.raises(ValueError):   # int64 indices
        gdn.fused_recurrent_gated_delta_rule_update(q, q, v, g, g, pool, idx.long())


# ---------------------------------------------------------------------------
# backward entry point
# ---------------------------------------------------------------------------
def _bcall(shape, ws=FAKE, ws_bytes=1 << 40, cu=None, ptrs=FAKE, dout=FAKE):
    lib = gdn.load_library()
    P = ctypes.c_void_p
    return lib.gdn_chunk_bwd(P(ptrs), P(ptrs), P(ptrs), P(ptrs), P(ptrs), P(dout) if dout else None, None,
                             1.0, 1, None, None if cu is None else P(cu), P(ptrs), P(ptrs), P(ptrs), P(ptrs),
                             P(ptrs), None, None if shape is None else ctypes.byref(shape), P(ws) if ws else None,
                             ws_bytes, None)


def test_backward_workspace_size():
    # equal-length: per chunk and value head 2 K V floats and three 64 x 64
    # matrices kept as their ten 16 x 16 blocks on and below the diagonal, per
    # token and value head 2 V + 2 K + 1 floats, N + 1 chunk offsets; each
    # region rounded up to 256 bytes
    tri = 10 * 16 * 16
    B, T, H, HV, K, V = 4, 4096, 16, 32, 128, 128
    got = gdn.gdn_chunk_bwd_workspace_bytes(gdn.make_shape(B, T, H, HV, K, V, B, gdn.GDN_BF16))
    chunks = B * T // 64
    want = 256 + 4 * (chunks * HV * (2 * K * V + 3 * tri) + B * T * HV * (2 * V + 2 * K + 1))
    assert want <= got <= want + 11 * 256
    # B == 1: slots for packed sequences, ceil(T/64) + N chunks, and the
    # longest-first order of the N sequences (N int32)
    g1 = gdn.gdn_chunk_bwd_workspace_bytes(gdn.make_shape(1, 1000, 2, 4, 64, 64, 7, gdn.GDN_F32))
    slots = (1000 + 63) // 64 + 7
    want1 = 4 * (slots * 4 * (2 * 64 * 64 + 3 * tri) + 1000 * 4 * (2 * 64 + 2 * 64 + 1) + 7)
    assert want1 <= g1 <= want1 + 13 * 256
    assert gdn.gdn_chunk_bwd_workspace_bytes(gdn.make_shape(1, 64, 2, 4, 96, 64, 1, 0)) == 0   # K unsupported


@pytest.mark.parametrize("shape,ws,ws_bytes,cu,want", [
    (None, FAKE, 1 << 40, None, -1),
    (gdn.make_shape(2, 64, 2, 4, 128, 128, 2, 0), None, 0, None, -5),          # no workspace
    (gdn.make_shape(2, 64, 2, 4, 128, 128, 2, 0), FAKE, 1024, None, -5),       # too small
    (gdn.make_shape(2, 64, 2, 4, 128, 128, 2, 0), FAKE + 16, 1 << 40, None, -5),   # misaligned
    (gdn.make_shape(2, 64, 2, 4, 128, 128, 3, 0), FAKE, 1 << 40, None, -2),    # N != B
    (gdn.make_shape(2, 64, 2, 4, 128, 128, 2, 0), FAKE, 1 << 40, FAKE, -2),    # B != 1 with cu_seqlens
    (gdn.make_shape(1, 64, 2, 3, 128, 128, 1, 0), FAKE, 1 << 40, None, -4),    # HV % H
    (gdn.make_shape(1, 64, 2, 4, 128, 128, 1, 5), FAKE, 1 << 40, None, -3),    # dtype
])
def test_backward_argument_errors(shape, ws, ws_bytes, cu, want):
    assert _bcall(shape, ws=ws, ws_bytes=ws_bytes, cu=cu) == want


def test_backward_null_and_misaligned_tensor_errors():
    s = gdn.make_shape(2, 64, 2, 4, 128, 128, 2, 0)
    assert _bcall(s, dout=0) == -1
    assert _bcall(s, ptrs=0) == -1
    assert _bcall(s, dout=FAKE + 8) == -7


def test_backward_wrapper_rejects_cpu_tensors_and_bad_shapes():
    import torch
    q = torch.zeros(1, 8, 2, 64)
    v = torch.zeros(1, 8, 4, 64)
    g = torch.zeros(1, 8, 4)
    with pytest.raises(ValueError):
        gdn.chunk_gated_delta_rule_bwd(q, q, v, g, g, v)          # CPU tensors: no CPU path
    with pytest.raises(ValueError):
        gdn.chunk_gated_delta_rule_bwd(q, q, v, g, g, v[:, :4])   # do shape
