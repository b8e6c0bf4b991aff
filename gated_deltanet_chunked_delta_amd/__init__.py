"""MI355X-native gated delta rule: chunked prefill and its backward pass,
fused recurrent decode and the gate computation.

The compute path is the C-ABI library ``libgdn.so`` (hand-written HIP kernels
for gfx950, declared in ``include/gdn.h``); this package only marshals
arguments to it.
"""
from ._binding import (EXPORTED, GDN_BF16, GDN_ERR_SCRATCH, GDN_F32, GDN_OK, GDN_STATIC_SCRATCH_BYTES, LIB_PATH, GdnError, chunk_gated_delta_rule,
                       chunk_gated_delta_rule_bwd, gdn_chunk_bwd, gdn_chunk_bwd_workspace_bytes,
                       fused_gdn_gating, fused_gdn_gating_bwd, fused_recurrent_gated_delta_rule_update, gdn_chunk_fwd,
                       gdn_chunk_fwd_noalloc,
                       gdn_chunk_fwd_gated, gdn_chunk_fwd_pool, gdn_chunk_fwd_workspace_bytes, gdn_decode_shape,
                       gdn_gates, gdn_gating, gdn_gating_bwd, gdn_gating_bwd_workspace_bytes,
                       gdn_profile_enable, gdn_profile_read, gdn_recurrent_update,
                       gdn_recurrent_update_gated, gdn_recurrent_update_pool, gdn_shape, gdn_state_pool,
                       gdn_status_str, load_library, make_decode_shape, make_gates, make_shape, make_state_pool)

__all__ = ["EXPORTED", "GDN_BF16", "GDN_ERR_SCRATCH", "GDN_F32", "GDN_OK", "GDN_STATIC_SCRATCH_BYTES", "LIB_PATH", "GdnError", "chunk_gated_delta_rule",
           "chunk_gated_delta_rule_bwd", "gdn_chunk_bwd", "gdn_chunk_bwd_workspace_bytes",
           "fused_gdn_gating", "fused_gdn_gating_bwd", "fused_recurrent_gated_delta_rule_update", "gdn_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_chunk_fwd_gated",
           "gdn_chunk_fwd_pool", "gdn_chunk_fwd_workspace_bytes", "gdn_decode_shape", "gdn_gates", "gdn_gating",
           "gdn_gating_bwd", "gdn_gating_bwd_workspace_bytes",
           "gdn_profile_enable", "gdn_profile_read", "gdn_recurrent_update", "gdn_recurrent_update_gated",
           "gdn_recurrent_update_pool", "gdn_shape", "gdn_state_pool", "gdn_status_str", "load_library",
           "make_decode_shape", "make_gates", "make_shape", "make_state_pool"]
