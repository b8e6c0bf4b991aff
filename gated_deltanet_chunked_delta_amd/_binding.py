"""ctypes binding of the C ABI in include/gdn.h.

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of libgdn.so.  There is no CPU path; if the library is missing or the
tensors are not on a GPU, the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_OK = 0
GDN_BF16 = 0
GDN_F32 = 1
GDN_ERR_SCRATCH = -8
GDN_STATIC_SCRATCH_BYTES = 64 << 20      # the static scratch of gdn_chunk_fwd_noalloc, per GPU
EXPORTED = ("gdn_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_chunk_fwd_gated", "gdn_chunk_fwd_pool", "gdn_chunk_fwd_workspace_bytes",
            "gdn_chunk_bwd", "gdn_chunk_bwd_workspace_bytes",
            "gdn_gating", "gdn_gating_bwd", "gdn_gating_bwd_workspace_bytes", "gdn_recurrent_update", "gdn_recurrent_update_gated", "gdn_recurrent_update_pool",
            "gdn_profile_enable", "gdn_profile_read", "gdn_status_str")

_DTYPES = {torch.bfloat16: GDN_BF16, torch.float32: GDN_F32}


class gdn_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("HV", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32),
                ("N", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class gdn_decode_shape(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("H", ctypes.c_int32), ("HV", ctypes.c_int32),
                ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("pool_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class gdn_gates(ctypes.Structure):
    _fields_ = [("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p), ("a", ctypes.c_void_p),
                ("b", ctypes.c_void_p)]


class gdn_state_pool(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("indices", ctypes.c_void_p), ("pool_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("read_initial", ctypes.c_int32)]


class GdnError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, status: int):
        self.status = status
        super().__init__(gdn_status_str(status))


_lib = None


def load_library(path: str = LIB_PATH):
    """Loads libgdn.so (once) and declares the exported signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build() "
                           "(or python gated_deltanet_chunked_delta_amd/build.py)")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.gdn_chunk_fwd_workspace_bytes.argtypes = [ctypes.POINTER(gdn_shape)]
    lib.gdn_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_chunk_fwd.argtypes = [P, P, P, P, P, ctypes.c_float, ctypes.c_int, P, P, P, P,
                                  ctypes.POINTER(gdn_shape), P, ctypes.c_size_t, P]
    lib.gdn_chunk_fwd.restype = ctypes.c_int
    lib.gdn_chunk_fwd_noalloc.argtypes = [P, P, P, P, P, ctypes.c_float, ctypes.c_int, P, P, P, P,
                                          ctypes.POINTER(gdn_shape), P]
    lib.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.gdn_chunk_bwd_workspace_bytes.argtypes = [ctypes.POINTER(gdn_shape)]
    lib.gdn_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_chunk_bwd.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_int, P, P, P, P, P, P, P, P,
                                  ctypes.POINTER(gdn_shape), P, ctypes.c_size_t, P]
    lib.gdn_chunk_bwd.restype = ctypes.c_int
    lib.gdn_recurrent_update.argtypes = [P, P, P, P, P, ctypes.c_float, ctypes.c_int, P, P, P,
                                         ctypes.POINTER(gdn_decode_shape), P]
    lib.gdn_recurrent_update.restype = ctypes.c_int
    G = ctypes.POINTER(gdn_gates)
    lib.gdn_chunk_fwd_gated.argtypes = [P, P, P, G, ctypes.c_float, ctypes.c_int, P, P, P, P,
                                        ctypes.POINTER(gdn_shape), P, ctypes.c_size_t, P]
    lib.gdn_chunk_fwd_gated.restype = ctypes.c_int
    lib.gdn_recurrent_update_gated.argtypes = [P, P, P, G, ctypes.c_float, ctypes.c_int, P, P, P,
                                               ctypes.POINTER(gdn_decode_shape), P]
    lib.gdn_recurrent_update_gated.restype = ctypes.c_int
    lib.gdn_gating.argtypes = [G, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P, P]
    lib.gdn_gating.restype = ctypes.c_int
    lib.gdn_gating_bwd_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32]
    lib.gdn_gating_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_gating_bwd.argtypes = [G, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P, P,
                                   ctypes.c_size_t, P]
    lib.gdn_gating_bwd.restype = ctypes.c_int
    SP = ctypes.POINTER(gdn_state_pool)
    lib.gdn_chunk_fwd_pool.argtypes = [P, P, P, P, P, G, ctypes.c_float, ctypes.c_int, SP, P, P,
                                       ctypes.POINTER(gdn_shape), P, ctypes.c_size_t, P]
    lib.gdn_chunk_fwd_pool.restype = ctypes.c_int
    lib.gdn_recurrent_update_pool.argtypes = [P, P, P, P, P, G, ctypes.c_float, ctypes.c_int, SP, P,
                                              ctypes.POINTER(gdn_decode_shape), P]
    lib.gdn_recurrent_update_pool.restype = ctypes.c_int
    lib.gdn_profile_enable.argtypes = [ctypes.c_int]
    lib.gdn_profile_enable.restype = ctypes.c_int
    lib.gdn_profile_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                     ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.gdn_profile_read.restype = ctypes.c_int
    lib.gdn_status_str.argtypes = [ctypes.c_int]
    lib.gdn_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def gdn_status_str(status: int) -> str:
    return load_library().gdn_status_str(int(status)).decode()


def gdn_profile_enable(enable: bool) -> int:
    """Starts (True) or stops (False) event timing of the library's kernels;
    either way the accumulated totals are cleared."""
    return int(load_library().gdn_profile_enable(int(bool(enable))))


def gdn_profile_read():
    """Returns {kernel name: (total ms, launches)} accumulated since enabling
    (synchronises on the recorded events)."""
    lib = load_library()
    n = int(lib.gdn_profile_read(0, None, None, None))
    names = (ctypes.c_char_p * n)()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    k = lib.gdn_profile_read(n, names, ms, cnt)
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(min(k, n))}


def make_shape(B, T, H, HV, K, V, N, dtype) -> gdn_shape:
    return gdn_shape(int(B), int(T), int(H), int(HV), int(K), int(V), int(N), int(dtype))


def gdn_chunk_fwd_workspace_bytes(shape: gdn_shape) -> int:
    return int(load_library().gdn_chunk_fwd_workspace_bytes(ctypes.byref(shape)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def gdn_chunk_fwd(q, k, v, g, beta, scale, use_l2norm, initial_state, cu_seqlens, out, final_state,
                  shape: gdn_shape, workspace, workspace_bytes=None, stream=None) -> int:
    """Direct call of the C entry point with tensors as device buffers.

    Returns the status code (0 = GDN_OK); does not raise on a bad status.
    ``stream`` is a raw hipStream_t handle (int) or None for torch's current
    stream on q's device.
    """
    lib = load_library()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return int(lib.gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                                 int(bool(use_l2norm)), _ptr(initial_state), _ptr(cu_seqlens), _ptr(out),
                                 _ptr(final_state), ctypes.byref(shape), _ptr(workspace),
                                 int(workspace_bytes), ctypes.c_void_p(int(stream))))


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, scale, use_l2norm, initial_state, cu_seqlens, out, final_state,
                          shape: gdn_shape, stream=None) -> int:
    """Direct call of the allocation-free forward entry point (gdn_chunk_fwd
    without a workspace: a split uses the library's static scratch); returns
    the status code.  ``stream`` as for gdn_chunk_fwd."""
    lib = load_library()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    return int(lib.gdn_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                                         int(bool(use_l2norm)), _ptr(initial_state), _ptr(cu_seqlens), _ptr(out),
                                         _ptr(final_state), ctypes.byref(shape), ctypes.c_void_p(int(stream))))


def _check(cond, msg):
    if not cond:
        raise ValueError(msg)


def chunk_gated_delta_rule(q, k, v, g=None, beta=None, scale=None, initial_state=None, output_final_state=True,
                           cu_seqlens=None, use_qk_l2norm_in_kernel=False, workspace=None, out=None,
                           final_state=None, A_log=None, dt_bias=None, a_raw=None, b_raw=None,
                           ssm_state_pool=None, ssm_state_indices=None, read_initial_state=True):
    """Forward chunked gated delta rule on the GPU.

    q, k [B,T,H,K] and v [B,T,HV,V] (bf16, or fp32 for the check mode);
    g, beta [B,T,HV] fp32; initial_state [N,HV,K,V] fp32 or None;
    cu_seqlens [N+1] int32 on the device or None.  Returns
    ``(o [B,T,HV,V], final_state [N,HV,K,V] fp32 or None)``.  ``scale=None``
    means 1/sqrt(K).  Optional preallocated ``workspace`` (uint8),
    ``out`` and ``final_state`` are used as given.

    Instead of g and beta, the raw gate inputs A_log, dt_bias [HV] fp32 and
    a_raw, b_raw [B,T,HV] (q's dtype) may be given; the kernel then computes
    g = -exp(A_log) softplus(a_raw + dt_bias) and beta = sigmoid(b_raw).

    With ``ssm_state_pool`` [P,HV,K,V] (float32 or bfloat16) and
    ``ssm_state_indices`` [N] int32, sequence n starts from slot
    ssm_state_indices[n] (from zero if ``read_initial_state`` is False) and its
    final state is written back to that slot in place; initial_state and
    final_state are then not used and the call returns ``(o, None)``.
    """
    _check(q.dim() == 4 and k.shape == q.shape, "q and k must be [B,T,H,K] of equal shape")
    B, T, H, K = q.shape
    _check(v.dim() == 4 and v.shape[:2] == (B, T), "v must be [B,T,HV,V]")
    HV, V = v.shape[2], v.shape[3]
    _check(q.dtype in _DTYPES and k.dtype == q.dtype and v.dtype == q.dtype,
           "q, k, v must share one dtype (bfloat16 or float32)")
    gated = g is None and beta is None
    _check(q.is_cuda, "tensors must be on a GPU device (there is no CPU path)")
    if gated:
        A_log, dt_bias, a_raw, b_raw = _gate_inputs(A_log, dt_bias, a_raw, b_raw, (B, T, HV), q.dtype, q.device)
    else:
        _check(g is not None and beta is not None and all(t is None for t in (A_log, dt_bias, a_raw, b_raw)),
               "give either g and beta or the raw gate inputs")
        _check(tuple(g.shape) == (B, T, HV) and g.dtype == torch.float32, "g must be float32 [B,T,HV]")
        _check(tuple(beta.shape) == (B, T, HV) and beta.dtype == torch.float32, "beta must be float32 [B,T,HV]")
    for name, t in (("k", k), ("v", v), ("g", g), ("beta", beta), ("initial_state", initial_state),
                    ("cu_seqlens", cu_seqlens)):
        _check(t is None or t.device == q.device, f"{name} must be on {q.device}")
    if cu_seqlens is not None:
        _check(B == 1, "cu_seqlens requires B == 1")
        _check(cu_seqlens.dim() == 1 and cu_seqlens.dtype == torch.int32, "cu_seqlens must be int32 [N+1]")
        N = cu_seqlens.shape[0] - 1
    else:
        N = B
    pooled = ssm_state_pool is not None
    if pooled:
        _check(initial_state is None and final_state is None,
               "with a state pool, initial and final states live in the pool")
        _check(ssm_state_pool.dim() == 4 and tuple(ssm_state_pool.shape[1:]) == (HV, K, V)
               and ssm_state_pool.dtype in _DTYPES and ssm_state_pool.is_contiguous()
               and ssm_state_pool.device == q.device,
               f"ssm_state_pool must be a contiguous float32/bfloat16 [P,{HV},{K},{V}] on {q.device}")
        _check(ssm_state_indices is not None and tuple(ssm_state_indices.shape) == (N,)
               and ssm_state_indices.dtype == torch.int32 and ssm_state_indices.device == q.device,
               f"ssm_state_indices must be int32 [{N}] on {q.device}")
    if initial_state is not None:
        _check(tuple(initial_state.shape) == (N, HV, K, V) and initial_state.dtype == torch.float32,
               f"initial_state must be float32 [{N},{HV},{K},{V}]")
    # buffers the caller hands in are written in place, so they must already
    # have the layout the kernels write
    if out is not None:
        _check(tuple(out.shape) == (B, T, HV, V) and out.dtype == q.dtype and out.is_contiguous()
               and out.device == q.device, f"out must be a contiguous {q.dtype} [{B},{T},{HV},{V}] on {q.device}")
    if final_state is not None and output_final_state:
        _check(tuple(final_state.shape) == (N, HV, K, V) and final_state.dtype == torch.float32
               and final_state.is_contiguous() and final_state.device == q.device,
               f"final_state must be a contiguous float32 [{N},{HV},{K},{V}] on {q.device}")
    if workspace is not None:
        _check(workspace.device == q.device and workspace.is_contiguous(),
               f"workspace must be a contiguous buffer on {q.device}")
    if cu_seqlens is not None:
        cu_seqlens = cu_seqlens.contiguous()
    if scale is None:
        scale = K ** -0.5
    q, k, v = (t.contiguous() for t in (q, k, v))
    if not gated:
        g, beta = g.contiguous(), beta.contiguous()
    if initial_state is not None:
        initial_state = initial_state.contiguous()
    shape = make_shape(B, T, H, HV, K, V, N, _DTYPES[q.dtype])
    need = gdn_chunk_fwd_workspace_bytes(shape)
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, T, HV, V), dtype=q.dtype, device=q.device)
    if pooled:
        pool = make_state_pool(ssm_state_pool, ssm_state_indices.contiguous(), read_initial_state)
        gates = make_gates(A_log, dt_bias, a_raw, b_raw) if gated else None
        st = gdn_chunk_fwd_pool(q, k, v, g, beta, gates, scale, use_qk_l2norm_in_kernel, pool, cu_seqlens, out,
                                shape, workspace)
        if st != GDN_OK:
            raise GdnError(st)
        return out, None
    if output_final_state and final_state is None:
        final_state = torch.empty((N, HV, K, V), dtype=torch.float32, device=q.device)
    if not output_final_state:
        final_state = None
    if gated:
        st = gdn_chunk_fwd_gated(q, k, v, make_gates(A_log, dt_bias, a_raw, b_raw), scale, use_qk_l2norm_in_kernel,
                                 initial_state, cu_seqlens, out, final_state, shape, workspace)
    else:
        st = gdn_chunk_fwd(q, k, v, g, beta, scale, use_qk_l2norm_in_kernel, initial_state, cu_seqlens, out,
                           final_state, shape, workspace)
    if st != GDN_OK:
        raise GdnError(st)
    return out, final_state


def gdn_chunk_bwd_workspace_bytes(shape: gdn_shape) -> int:
    return int(load_library().gdn_chunk_bwd_workspace_bytes(ctypes.byref(shape)))


def gdn_chunk_bwd(q, k, v, g, beta, dout, dht, scale, use_l2norm, initial_state, cu_seqlens, dq, dk, dv, dg,
                  dbeta, dh0, shape: gdn_shape, workspace, workspace_bytes=None, stream=None) -> int:
    """Direct call of the C backward entry point; returns the status code."""
    lib = load_library()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return int(lib.gdn_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(dout), _ptr(dht),
                                 float(scale), int(bool(use_l2norm)), _ptr(initial_state), _ptr(cu_seqlens),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0),
                                 ctypes.byref(shape), _ptr(workspace), int(workspace_bytes),
                                 ctypes.c_void_p(int(stream))))


def chunk_gated_delta_rule_bwd(q, k, v, g, beta, do, dht=None, scale=None, initial_state=None, cu_seqlens=None,
                               use_qk_l2norm_in_kernel=False, output_dh0=True, workspace=None):
    """Backward pass of ``chunk_gated_delta_rule`` (g / beta form) on the GPU.

    Takes the forward inputs, ``do`` (gradient of the output, q's dtype and
    [B,T,HV,V]) and ``dht`` (gradient of the final state, float32
    [N,HV,K,V], or None when the final state is unused).  Returns
    ``(dq, dk, dv, dg, dbeta, dh0)``: dq, dk, dv in q's dtype and shapes of
    q, k, v; dg, dbeta float32 [B,T,HV]; dh0 float32 [N,HV,K,V] (None when
    ``output_dh0`` is False).  A preallocated uint8 ``workspace`` of
    gdn_chunk_bwd_workspace_bytes bytes may be given.
    """
    _check(q.dim() == 4 and k.shape == q.shape, "q and k must be [B,T,H,K] of equal shape")
    B, T, H, K = q.shape
    _check(v.dim() == 4 and v.shape[:2] == (B, T), "v must be [B,T,HV,V]")
    HV, V = v.shape[2], v.shape[3]
    _check(q.dtype in _DTYPES and k.dtype == q.dtype and v.dtype == q.dtype and do.dtype == q.dtype,
           "q, k, v, do must share one dtype (bfloat16 or float32)")
    _check(q.is_cuda, "tensors must be on a GPU device (there is no CPU path)")
    _check(tuple(do.shape) == (B, T, HV, V), "do must have v's shape")
    _check(tuple(g.shape) == (B, T, HV) and g.dtype == torch.float32, "g must be float32 [B,T,HV]")
    _check(tuple(beta.shape) == (B, T, HV) and beta.dtype == torch.float32, "beta must be float32 [B,T,HV]")
    for name, t in (("k", k), ("v", v), ("g", g), ("beta", beta), ("do", do), ("dht", dht),
                    ("initial_state", initial_state), ("cu_seqlens", cu_seqlens)):
        _check(t is None or t.device == q.device, f"{name} must be on {q.device}")
    if cu_seqlens is not None:
        _check(B == 1, "cu_seqlens requires B == 1")
        _check(cu_seqlens.dim() == 1 and cu_seqlens.dtype == torch.int32, "cu_seqlens must be int32 [N+1]")
        N = cu_seqlens.shape[0] - 1
    else:
        N = B
    for name, t in (("initial_state", initial_state), ("dht", dht)):
        _check(t is None or (tuple(t.shape) == (N, HV, K, V) and t.dtype == torch.float32),
               f"{name} must be float32 [{N},{HV},{K},{V}]")
    if scale is None:
        scale = K ** -0.5
    q, k, v, g, beta, do = (t.contiguous() for t in (q, k, v, g, beta, do))
    initial_state = None if initial_state is None else initial_state.contiguous()
    dht = None if dht is None else dht.contiguous()
    shape = make_shape(B, T, H, HV, K, V, N, _DTYPES[q.dtype])
    need = gdn_chunk_bwd_workspace_bytes(shape)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty((B, T, HV), dtype=torch.float32, device=q.device)
    dbeta = torch.empty_like(dg)
    dh0 = torch.empty((N, HV, K, V), dtype=torch.float32, device=q.device) if output_dh0 else None
    st = gdn_chunk_bwd(q, k, v, g, beta, do, dht, scale, use_qk_l2norm_in_kernel, initial_state, cu_seqlens, dq,
                       dk, dv, dg, dbeta, dh0, shape, workspace)
    if st != GDN_OK:
        raise GdnError(st)
    return dq, dk, dv, dg, dbeta, dh0


def make_decode_shape(N, H, HV, K, V, pool_size, dtype) -> gdn_decode_shape:
    return gdn_decode_shape(int(N), int(H), int(HV), int(K), int(V), int(pool_size), int(dtype))


def gdn_recurrent_update(q, k, v, g, beta, scale, use_l2norm, state_pool, state_indices, out,
                         shape: gdn_decode_shape, stream=None) -> int:
    """Direct call of the C decode entry point; returns the status code."""
    lib = load_library()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    return int(lib.gdn_recurrent_update(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                                        int(bool(use_l2norm)), _ptr(state_pool), _ptr(state_indices),
                                        _ptr(out), ctypes.byref(shape), ctypes.c_void_p(int(stream))))


def fused_recurrent_gated_delta_rule_update(q, k, v, g, beta, state_pool, state_indices, scale=None,
                                            use_qk_l2norm_in_kernel=False, out=None, A_log=None, dt_bias=None,
                                            a_raw=None, b_raw=None):
    """One decode step per sequence with an in-place, pool-indexed state.

    q, k [N,H,K] or [N,1,H,K]; v [N,HV,V] or [N,1,HV,V] (bf16, or fp32 for the
    check mode); g, beta [N,HV] or [N,1,HV] fp32; state_pool [P,HV,K,V] fp32
    or bf16 (rounded to nearest even when stored), updated in place; state_indices [N] int32 on the device (an entry outside
    [0, P), e.g. -1, marks a padding row: its slot is untouched and its output
    row is zero).  Returns o with v's shape.

    With g = beta = None, the raw gate inputs A_log, dt_bias [HV] fp32 and
    a_raw, b_raw [N,HV] or [N,1,HV] (q's dtype) give the gates in the kernel.
    """
    squeeze = q.dim() == 4
    if squeeze:
        _check(q.shape[1] == 1 and k.shape == q.shape and v.dim() == 4 and v.shape[1] == 1,
               "decode takes one token per sequence: [N,1,...] layouts need T == 1")
    qs, ks, vs = (t.reshape(t.shape[0], t.shape[-2], t.shape[-1]) for t in (q, k, v))
    N, H, K = qs.shape
    HV, V = vs.shape[1], vs.shape[2]
    _check(ks.shape == qs.shape and vs.shape[0] == N, "q, k must be [N,H,K] and v [N,HV,V]")
    _check(qs.dtype in _DTYPES and ks.dtype == qs.dtype and vs.dtype == qs.dtype,
           "q, k, v must share one dtype (bfloat16 or float32)")
    gated = g is None and beta is None
    if gated:
        A_log, dt_bias, a_raw, b_raw = _gate_inputs(A_log, dt_bias, a_raw, b_raw, (N, HV), qs.dtype, qs.device)
        gs = bs = None
    else:
        _check(g is not None and beta is not None and all(t is None for t in (A_log, dt_bias, a_raw, b_raw)),
               "give either g and beta or the raw gate inputs")
        gs, bs = g.reshape(N, HV), beta.reshape(N, HV)
        _check(tuple(gs.shape) == (N, HV) and gs.dtype == torch.float32, "g must be float32 [N,HV]")
        _check(tuple(bs.shape) == (N, HV) and bs.dtype == torch.float32, "beta must be float32 [N,HV]")
    _check(state_pool.dim() == 4 and tuple(state_pool.shape[1:]) == (HV, K, V)
           and state_pool.dtype in _DTYPES and state_pool.is_contiguous(),
           f"state_pool must be a contiguous float32 or bfloat16 [P,{HV},{K},{V}]")
    _check(tuple(state_indices.shape) == (N,) and state_indices.dtype == torch.int32,
           "state_indices must be int32 [N]")
    _check(qs.is_cuda, "tensors must be on a GPU device (there is no CPU path)")
    for name, t in (("k", ks), ("v", vs), ("g", gs), ("beta", bs), ("state_pool", state_pool),
                    ("state_indices", state_indices)):
        _check(t is None or t.device == qs.device, f"{name} must be on {qs.device}")
    if scale is None:
        scale = K ** -0.5
    qs, ks, vs, idx = (t.contiguous() for t in (qs, ks, vs, state_indices))
    if not gated:
        gs, bs = gs.contiguous(), bs.contiguous()
    if out is None:
        out = torch.empty((N, HV, V), dtype=qs.dtype, device=qs.device)
    shape = make_decode_shape(N, H, HV, K, V, state_pool.shape[0], _DTYPES[qs.dtype])
    if state_pool.dtype == torch.bfloat16:
        gates = make_gates(A_log, dt_bias, a_raw, b_raw) if gated else None
        st = gdn_recurrent_update_pool(qs, ks, vs, gs, bs, gates, scale, use_qk_l2norm_in_kernel,
                                       make_state_pool(state_pool, idx), out, shape)
    elif gated:
        st = gdn_recurrent_update_gated(qs, ks, vs, make_gates(A_log, dt_bias, a_raw, b_raw), scale,
                                        use_qk_l2norm_in_kernel, state_pool, idx, out, shape)
    else:
        st = gdn_recurrent_update(qs, ks, vs, gs, bs, scale, use_qk_l2norm_in_kernel, state_pool, idx, out,
                                  shape)
    if st != GDN_OK:
        raise GdnError(st)
    return out.reshape(v.shape) if squeeze else out


def make_gates(A_log, dt_bias, a, b) -> gdn_gates:
    """The raw gate inputs as a gdn_gates struct of device pointers (the
    tensors must stay alive while the struct is in use)."""
    return gdn_gates(*(None if t is None else t.data_ptr() for t in (A_log, dt_bias, a, b)))


def _stream(t, stream):
    return ctypes.c_void_p(int(torch.cuda.current_stream(t.device).cuda_stream if stream is None else stream))


def gdn_gating(gates: gdn_gates, rows, HV, dtype, g, beta, stream=None, device=None) -> int:
    """Direct call of the C gating entry point; returns the status code."""
    lib = load_library()
    if stream is None:
        stream = torch.cuda.current_stream(device if device is not None else g.device).cuda_stream
    return int(lib.gdn_gating(ctypes.byref(gates), int(rows), int(HV), int(dtype), _ptr(g), _ptr(beta),
                              ctypes.c_void_p(int(stream))))


def gdn_gating_bwd_workspace_bytes(rows, HV) -> int:
    return int(load_library().gdn_gating_bwd_workspace_bytes(int(rows), int(HV)))


def gdn_gating_bwd(gates: gdn_gates, rows, HV, dtype, dg, dbeta, da, db, dA_log, ddt_bias, workspace,
                   workspace_bytes=None, stream=None, device=None) -> int:
    """Direct call of the C gate-gradient entry point; returns the status code."""
    lib = load_library()
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(device if device is not None else dA_log.device).cuda_stream
    return int(lib.gdn_gating_bwd(ctypes.byref(gates), int(rows), int(HV), int(dtype), _ptr(dg), _ptr(dbeta),
                                  _ptr(da), _ptr(db), _ptr(dA_log), _ptr(ddt_bias), _ptr(workspace),
                                  int(workspace_bytes), ctypes.c_void_p(int(stream))))


def gdn_chunk_fwd_gated(q, k, v, gates: gdn_gates, scale, use_l2norm, initial_state, cu_seqlens, out,
                        final_state, shape: gdn_shape, workspace, workspace_bytes=None, stream=None) -> int:
    """Direct call of the C prefill entry point with in-kernel gating."""
    lib = load_library()
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return int(lib.gdn_chunk_fwd_gated(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(gates), float(scale),
                                       int(bool(use_l2norm)), _ptr(initial_state), _ptr(cu_seqlens), _ptr(out),
                                       _ptr(final_state), ctypes.byref(shape), _ptr(workspace),
                                       int(workspace_bytes), _stream(q, stream)))


def gdn_recurrent_update_gated(q, k, v, gates: gdn_gates, scale, use_l2norm, state_pool, state_indices, out,
                               shape: gdn_decode_shape, stream=None) -> int:
    """Direct call of the C decode entry point with in-kernel gating."""
    lib = load_library()
    return int(lib.gdn_recurrent_update_gated(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(gates), float(scale),
                                              int(bool(use_l2norm)), _ptr(state_pool), _ptr(state_indices),
                                              _ptr(out), ctypes.byref(shape), _stream(q, stream)))


def _gate_inputs(A_log, dt_bias, a, b, rows_shape, io_dtype, device):
    """Checks the raw gate inputs against a [rows..., HV] layout and returns
    contiguous copies (a, b reshaped to rows x HV)."""
    HV = rows_shape[-1]
    _check(all(t is not None for t in (A_log, dt_bias, a, b)),
           "in-kernel gating needs all of A_log, dt_bias, a_raw, b_raw")
    _check(tuple(A_log.shape) == (HV,) and tuple(dt_bias.shape) == (HV,) and A_log.dtype == torch.float32
           and dt_bias.dtype == torch.float32, f"A_log and dt_bias must be float32 [{HV}]")
    n = 1
    for d in rows_shape:
        n *= d
    _check(a.numel() == n and b.numel() == n and a.dtype == io_dtype and b.dtype == io_dtype,
           f"a_raw and b_raw must hold {tuple(rows_shape)} elements of q's dtype")
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias), ("a_raw", a), ("b_raw", b)):
        _check(t.device == device, f"{name} must be on {device}")
    return A_log.contiguous(), dt_bias.contiguous(), a.contiguous(), b.contiguous()


def fused_gdn_gating(A_log, a, b, dt_bias):
    """g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b) on the GPU.

    A_log, dt_bias [HV] float32; a, b [..., HV] bfloat16 or float32.
    Returns (g, beta), float32 with a's shape."""
    _check(a.is_cuda, "tensors must be on a GPU device (there is no CPU path)")
    _check(a.dtype in _DTYPES and b.dtype == a.dtype and tuple(b.shape) == tuple(a.shape) and a.dim() >= 1,
           "a and b must share one shape [..., HV] and dtype (bfloat16 or float32)")
    HV = a.shape[-1]
    A_log, dt_bias, ac, bc = _gate_inputs(A_log, dt_bias, a, b, tuple(a.shape), a.dtype, a.device)
    g = torch.empty(a.shape, dtype=torch.float32, device=a.device)
    beta = torch.empty_like(g)
    gates = make_gates(A_log, dt_bias, ac, bc)
    st = gdn_gating(gates, a.numel() // HV, HV, _DTYPES[a.dtype], g, beta)
    if st != GDN_OK:
        raise GdnError(st)
    return g, beta


def fused_gdn_gating_bwd(A_log, a, b, dt_bias, dg, dbeta):
    """Gradients of the gate inputs of fused_gdn_gating, given dg and dbeta
    (float32, a's shape; as chunk_gated_delta_rule_bwd returns them).

    Returns (da, db, dA_log, ddt_bias): da, db with a's shape and dtype,
    dA_log, ddt_bias [HV] float32."""
    _check(a.is_cuda, "tensors must be on a GPU device (there is no CPU path)")
    _check(a.dtype in _DTYPES and b.dtype == a.dtype and tuple(b.shape) == tuple(a.shape) and a.dim() >= 1,
           "a and b must share one shape [..., HV] and dtype (bfloat16 or float32)")
    _check(dg.dtype == torch.float32 and dbeta.dtype == torch.float32 and tuple(dg.shape) == tuple(a.shape)
           and tuple(dbeta.shape) == tuple(a.shape), "dg and dbeta must be float32 with a's shape")
    HV = a.shape[-1]
    A_log, dt_bias, ac, bc = _gate_inputs(A_log, dt_bias, a, b, tuple(a.shape), a.dtype, a.device)
    dg, dbeta = dg.contiguous(), dbeta.contiguous()
    rows = a.numel() // HV
    da, db = torch.empty_like(ac), torch.empty_like(bc)
    dA_log = torch.empty(HV, dtype=torch.float32, device=a.device)
    ddt_bias = torch.empty_like(dA_log)
    ws = torch.empty(max(gdn_gating_bwd_workspace_bytes(rows, HV), 1), dtype=torch.uint8, device=a.device)
    st = gdn_gating_bwd(make_gates(A_log, dt_bias, ac, bc), rows, HV, _DTYPES[a.dtype], dg, dbeta, da, db,
                        dA_log, ddt_bias, ws)
    if st != GDN_OK:
        raise GdnError(st)
    return da, db, dA_log, ddt_bias


def make_state_pool(data, indices, read_initial=True) -> gdn_state_pool:
    """A gdn_state_pool struct over a [P,HV,K,V] tensor (float32 or bfloat16)
    and [N] int32 slot indices (the tensors must stay alive while it is used)."""
    return gdn_state_pool(data.data_ptr(), indices.data_ptr(), int(data.shape[0]), _DTYPES[data.dtype],
                          int(bool(read_initial)))


def gdn_chunk_fwd_pool(q, k, v, g, beta, gates, scale, use_l2norm, pool: gdn_state_pool, cu_seqlens, out,
                       shape: gdn_shape, workspace, workspace_bytes=None, stream=None) -> int:
    """Direct call of the C prefill entry point with a state pool (gates may
    be None: g and beta are then used)."""
    lib = load_library()
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return int(lib.gdn_chunk_fwd_pool(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      None if gates is None else ctypes.byref(gates), float(scale),
                                      int(bool(use_l2norm)), ctypes.byref(pool), _ptr(cu_seqlens), _ptr(out),
                                      ctypes.byref(shape), _ptr(workspace), int(workspace_bytes),
                                      _stream(q, stream)))


def gdn_recurrent_update_pool(q, k, v, g, beta, gates, scale, use_l2norm, pool: gdn_state_pool, out,
                              shape: gdn_decode_shape, stream=None) -> int:
    """Direct call of the C decode entry point with a state pool."""
    lib = load_library()
    return int(lib.gdn_recurrent_update_pool(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                             None if gates is None else ctypes.byref(gates), float(scale),
                                             int(bool(use_l2norm)), ctypes.byref(pool), _ptr(out),
                                             ctypes.byref(shape), _stream(q, stream)))
