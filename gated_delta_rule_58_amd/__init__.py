"""MI355X (gfx950) gated-delta-rule library: Python front end of libgdn.so.

    from gated_delta_rule_58_amd import chunk_fwd, step
    o, S_T = chunk_fwd(q, k, v, log_alpha, beta, S0)    # chunkwise forward
    o = step(q_t, k_t, v_t, log_alpha_t, beta_t, S)      # decode, S in place

The rule is S_t = S_{t-1}(alpha_t (I - beta_t k_t k_t^T)) + beta_t v_t k_t^T
with the read-out o_t = S_t q_t ("Gated Delta Networks: Improving Mamba2 with
Delta Rule", research-map summary, section "Approach").  All arithmetic runs
in the HIP kernels of libgdn.so; see include/gdn.h for the C ABI.
"""
from ._binding import (GDN_BF16, GDN_F32, GdnError, chunk_bwd,  # noqa: F401
                       chunk_bwd_workspace_size, chunk_fwd, chunk_fwd_workspace_size,
                       gdn2_fwd, gdn2_fwd_workspace_size, kda_fwd, kda_fwd_noalloc,
                       kda_fwd_noalloc_max_workspace, kda_fwd_workspace_size, lib,
                       step, version)

__all__ = ["chunk_fwd", "chunk_bwd", "step", "chunk_fwd_workspace_size",
           "chunk_bwd_workspace_size", "kda_fwd", "kda_fwd_workspace_size", "kda_fwd_noalloc",
           "kda_fwd_noalloc_max_workspace", "gdn2_fwd",
           "gdn2_fwd_workspace_size", "version", "lib", "GdnError", "GDN_F32", "GDN_BF16"]
