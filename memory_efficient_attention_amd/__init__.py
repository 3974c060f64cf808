"""Fused memory-efficient attention (forward and backward) for AMD Instinct MI355X (gfx950).

The computation lives in the HIP library ``libmea.so`` (C ABI: include/mea.h);
this package is its Python binding.  ``_native`` wraps the C entry points
one to one; ``api`` adds the xFormers-style call with block-diagonal masks.
"""
from . import _native
from ._native import (mea_abi_version, mea_bwd, mea_bwd_workspace_size, mea_default_chunk_keys, mea_fwd,
                      mea_fwd_fp8, mea_fwd_fp8_workspace_size, mea_fwd_paged, mea_fwd_paged_fp8, mea_fwd_splitkv,
                      mea_fwd_workspace_size, mea_last_error, mea_status_string, mea_swiglu_ffn)
from .api import (BlockDiagonalCausalMask, BlockDiagonalMask, MeaError, attention_backward_packed,
                  attention_packed, attention_packed_fp8, attention_paged, attention_paged_fp8,
                  memory_efficient_attention, swiglu_ffn)

__all__ = [
    "BlockDiagonalMask", "BlockDiagonalCausalMask", "MeaError", "attention_packed",
    "attention_paged", "attention_backward_packed", "memory_efficient_attention", "mea_fwd",
    "mea_fwd_splitkv", "mea_fwd_paged", "mea_fwd_workspace_size", "mea_bwd", "mea_bwd_workspace_size",
    "attention_packed_fp8", "attention_paged_fp8", "mea_fwd_fp8", "mea_fwd_paged_fp8", "mea_fwd_fp8_workspace_size",
    "swiglu_ffn", "mea_swiglu_ffn",
    "mea_default_chunk_keys", "mea_status_string", "mea_last_error", "mea_abi_version",
]
