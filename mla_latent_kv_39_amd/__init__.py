"""MLA decode over a paged latent cache on MI355X (gfx950).

The hot path lives in libmla.so (HIP kernels behind the C ABI of
include/mla.h); `binding` marshals torch tensors into that ABI and `runner`
drives one decode step on device-resident inputs.
"""
from .binding import (LatentCache, MlaError, PreparedStep, MLA_CACHE_BF16, MLA_CACHE_FP8_E4M3, ROPE_BASE, mla_absorb_output,
                      mla_absorb_query, mla_cache_append, mla_check_indices, mla_combine, mla_decode,
                      mla_decode_noalloc, mla_init, mla_kv_project, mla_kv_project_split, mla_kv_project_splits,
                      mla_num_splits_hint, mla_partial_lse_bytes, mla_partial_out_bytes, mla_version, status_string)

__all__ = ["LatentCache", "MlaError", "PreparedStep", "MLA_CACHE_BF16", "MLA_CACHE_FP8_E4M3", "ROPE_BASE", "mla_absorb_output",
           "mla_absorb_query", "mla_cache_append", "mla_check_indices", "mla_combine", "mla_decode",
           "mla_decode_noalloc", "mla_init", "mla_kv_project", "mla_kv_project_split", "mla_kv_project_splits",
           "mla_num_splits_hint", "mla_partial_lse_bytes",
           "mla_partial_out_bytes", "mla_version", "status_string"]
