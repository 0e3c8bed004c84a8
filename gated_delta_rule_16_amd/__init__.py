"""Chunkwise gated delta rule forward for AMD MI355X (gfx950).

The compute path is the HIP library ``libgdn.so`` (kernels and C ABI under
``csrc/``, declared in ``include/gdn.h``); this package binds it with ctypes
and supplies seeded synthetic inputs (``inputs``).  Importing the package does
not load the library; the first call does, and fails loudly if it is missing.
"""
from .binding import (GDN_BF16, GDN_F32, GDN_RULE_DELTA, GDN_RULE_GLA, GDN_RULE_MAMBA2,
                      GdnError, LIB_PATH, gdn_chunk_fwd, gdn_chunk_fwd_noalloc,
                      gdn_chunk_fwd_auto_span_chunks, gdn_chunk_fwd_profiled, gdn_chunk_fwd_split,
                      gdn_chunk_fwd_split_workspace_bytes, gdn_chunk_fwd_supported,
                      gdn_chunk_fwd_workspace_bytes, gdn_gla_chunk_fwd, gdn_mamba2_chunk_fwd, gdn_recurrent_step, gdn_rule_chunk_fwd_profiled,
                      gdn_rule_supported, gdn_rule_workspace_bytes, gdn_status_string,
                      load_library)

__all__ = ["GDN_BF16", "GDN_F32", "GDN_RULE_DELTA", "GDN_RULE_GLA", "GDN_RULE_MAMBA2", "GdnError",
           "LIB_PATH", "gdn_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_chunk_fwd_profiled",
           "gdn_chunk_fwd_auto_span_chunks", "gdn_chunk_fwd_split", "gdn_chunk_fwd_split_workspace_bytes",
           "gdn_chunk_fwd_supported", "gdn_chunk_fwd_workspace_bytes", "gdn_gla_chunk_fwd",
           "gdn_mamba2_chunk_fwd",
           "gdn_recurrent_step", "gdn_rule_chunk_fwd_profiled", "gdn_rule_supported",
           "gdn_rule_workspace_bytes", "gdn_status_string", "load_library"]
