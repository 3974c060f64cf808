"""ctypes binding of the C ABI in ``include/mea.h`` (argument marshalling only).

Every function here has the name and the argument order of the C entry point
it wraps and passes plain integers (device addresses, sizes) straight
through.  Loading fails loudly if ``libmea.so`` has not been built: there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "MEA_OK", "MEA_ERR_INVALID", "MEA_ERR_UNSUPPORTED", "MEA_ERR_HIP", "MEA_F16", "MEA_BF16",
    "EXPORTED_SYMBOLS", "library_path", "load", "mea_fwd", "mea_fwd_mixed", "mea_fwd_mixed_workspace_size",
    "mea_fwd_noalloc", "mea_fwd_splitkv", "mea_fwd_paged",
    "mea_fwd_workspace_size", "mea_default_chunk_keys", "mea_bwd", "mea_bwd_workspace_size",
    "mea_fwd_fp8", "mea_fwd_paged_fp8", "mea_fwd_fp8_workspace_size", "mea_swiglu_ffn", "mea_status_string",
    "mea_last_error", "mea_abi_version",
]

MEA_OK, MEA_ERR_INVALID, MEA_ERR_UNSUPPORTED, MEA_ERR_HIP = 0, 1, 2, 3
MEA_F16, MEA_BF16 = 0, 1

EXPORTED_SYMBOLS = (
    "mea_fwd", "mea_fwd_mixed", "mea_fwd_mixed_workspace_size", "mea_fwd_noalloc", "mea_fwd_splitkv", "mea_fwd_paged", "mea_fwd_workspace_size", "mea_default_chunk_keys",
    "mea_bwd", "mea_bwd_workspace_size", "mea_fwd_fp8", "mea_fwd_paged_fp8", "mea_fwd_fp8_workspace_size",
    "mea_swiglu_ffn", "mea_status_string", "mea_last_error", "mea_abi_version",
)

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_lock = threading.Lock()
_lib = None

_i32, _sz, _vp, _f32 = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_FWD_ARGS = [_vp, _vp, _vp, _vp, _vp,                # q k v out lse
             _vp, _vp, _i32, _i32, _i32, _i32, _i32,  # seqstart_q seqstart_k num_seqs total_q total_k max_q max_k
             _i32, _i32, _i32, _i32, _i32,      # Hq Hkv D dtype causal
             _vp, _f32, _vp, _sz, _vp]          # slopes scale workspace workspace_bytes stream


_PAGED_ARGS = [_vp, _vp, _vp, _vp, _vp,                # q k_cache v_cache out lse
               _vp, _vp, _vp,                          # seqstart_q seqstart_k block_table
               _i32, _i32, _i32, _i32, _i32,           # num_seqs total_q total_k max_q max_k
               _i32, _i32, _i32,                       # page_size num_pages max_blocks
               _i32, _i32, _i32, _i32, _i32,           # Hq Hkv D dtype causal
               _vp, _f32, _vp, _sz, _vp]               # slopes scale workspace workspace_bytes stream


_BWD_ARGS = [_vp, _vp, _vp, _vp, _vp, _vp,            # q k v out lse dout
             _vp, _vp, _vp,                          # dq dk dv
             _vp, _vp, _i32, _i32, _i32, _i32, _i32,  # seqstart_q seqstart_k num_seqs total_q total_k max_q max_k
             _i32, _i32, _i32, _i32, _i32,           # Hq Hkv D dtype causal
             _vp, _f32, _vp, _sz, _vp]               # slopes scale workspace workspace_bytes stream


_FP8_ARGS = [_vp, _vp, _vp, _f32, _f32, _f32, _vp, _vp,   # q k v q_scale k_scale v_scale out lse
             _vp, _vp, _i32, _i32, _i32, _i32, _i32,      # seqstart_q seqstart_k num_seqs total_q total_k max_q max_k
             _i32, _i32, _i32, _i32, _i32,                # Hq Hkv D out_dtype causal
             _vp, _f32, _vp, _sz, _vp]                    # slopes scale workspace workspace_bytes stream


_PAGED_FP8_ARGS = [_vp, _vp, _vp, _f32, _f32, _f32, _vp, _vp,   # q k_cache v_cache q/k/v_scale out lse
                   _vp, _vp, _vp,                               # seqstart_q seqstart_k block_table
                   _i32, _i32, _i32, _i32, _i32,                # num_seqs total_q total_k max_q max_k
                   _i32, _i32, _i32,                            # page_size num_pages max_blocks
                   _i32, _i32, _i32, _i32, _i32,                # Hq Hkv D out_dtype causal
                   _vp, _f32, _vp, _sz, _vp]                    # slopes scale workspace workspace_bytes stream


def library_path() -> str:
    return os.environ.get("MEA_LIBRARY", os.path.join(_PKG_DIR, "libmea.so"))


def load() -> ctypes.CDLL:
    """Load ``libmea.so`` (once).  Raises if it is missing or incomplete."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"HIP library {path} is not built; run `python -m memory_efficient_attention_amd.build` "
                "(there is no CPU fallback)")
        lib = ctypes.CDLL(path)
        lib.mea_fwd.argtypes = _FWD_ARGS
        lib.mea_fwd.restype = ctypes.c_int
        lib.mea_fwd_mixed.argtypes = _FWD_ARGS[:12] + [_i32] * 4 + _FWD_ARGS[12:]
        lib.mea_fwd_mixed.restype = ctypes.c_int
        lib.mea_fwd_mixed_workspace_size.argtypes = [_i32] * 10
        lib.mea_fwd_mixed_workspace_size.restype = _sz
        lib.mea_fwd_noalloc.argtypes = _FWD_ARGS[:19] + [_vp]   # no workspace, workspace_bytes
        lib.mea_fwd_noalloc.restype = ctypes.c_int
        lib.mea_fwd_splitkv.argtypes = _FWD_ARGS + [_i32]
        lib.mea_fwd_splitkv.restype = ctypes.c_int
        lib.mea_fwd_paged.argtypes = _PAGED_ARGS
        lib.mea_fwd_paged.restype = ctypes.c_int
        lib.mea_fwd_workspace_size.argtypes = [_i32] * 8
        lib.mea_fwd_workspace_size.restype = _sz
        lib.mea_default_chunk_keys.argtypes = [_i32] * 3
        lib.mea_default_chunk_keys.restype = _i32
        lib.mea_bwd.argtypes = _BWD_ARGS
        lib.mea_bwd.restype = ctypes.c_int
        lib.mea_bwd_workspace_size.argtypes = [_i32] * 6
        lib.mea_bwd_workspace_size.restype = _sz
        lib.mea_fwd_fp8.argtypes = _FP8_ARGS
        lib.mea_fwd_fp8.restype = ctypes.c_int
        lib.mea_fwd_paged_fp8.argtypes = _PAGED_FP8_ARGS
        lib.mea_fwd_paged_fp8.restype = ctypes.c_int
        lib.mea_fwd_fp8_workspace_size.argtypes = [_i32] * 7
        lib.mea_fwd_fp8_workspace_size.restype = _sz
        lib.mea_swiglu_ffn.argtypes = [_vp] * 6 + [_i32, _i32, _i32, _i32, _vp]
        lib.mea_swiglu_ffn.restype = ctypes.c_int
        lib.mea_status_string.argtypes = [ctypes.c_int]
        lib.mea_status_string.restype = ctypes.c_char_p
        lib.mea_last_error.argtypes = []
        lib.mea_last_error.restype = ctypes.c_char_p
        lib.mea_abi_version.argtypes = []
        lib.mea_abi_version.restype = _i32
        _lib = lib
        return lib


def mea_fwd(q, k, v, out, lse, seqstart_q, seqstart_k, num_seqs, total_q, total_k, max_seqlen_q,
            max_seqlen_k, Hq, Hkv, D, dtype, causal, alibi_slopes, scale, workspace,
            workspace_bytes, stream) -> int:
    return load().mea_fwd(q, k, v, out, lse, seqstart_q, seqstart_k, num_seqs, total_q, total_k,
                          max_seqlen_q, max_seqlen_k, Hq, Hkv, D, dtype, causal, alibi_slopes,
                          scale, workspace, workspace_bytes, stream)


def mea_fwd_mixed(q, k, v, out, lse, seqstart_q, seqstart_k, num_seqs, total_q, total_k, max_seqlen_q,
                  max_seqlen_k, num_prefill_seqs, prefill_total_q, prefill_total_k, decode_max_seqlen_k, Hq, Hkv, D,
                  dtype, causal, alibi_slopes, scale, workspace, workspace_bytes, stream) -> int:
    return load().mea_fwd_mixed(q, k, v, out, lse, seqstart_q, seqstart_k, num_seqs, total_q, total_k,
                                max_seqlen_q, max_seqlen_k, num_prefill_seqs, prefill_total_q, prefill_total_k,
                                decode_max_seqlen_k, Hq, Hkv, D, dtype, causal, alibi_slopes, scale, workspace,
                                workspace_bytes, stream)


def mea_fwd_mixed_workspace_size(num_seqs, total_k, max_seqlen_q, max_seqlen_k, num_prefill_seqs, prefill_total_k,
                                 decode_max_seqlen_k, Hq, Hkv, D) -> int:
    return load().mea_fwd_mixed_workspace_size(num_seqs, total_k, max_seqlen_q, max_seqlen_k, num_prefill_seqs,
                                               prefill_total_k, decode_max_seqlen_k, Hq, Hkv, D)


def mea_fwd_noalloc(q, k, v, out, lse, seqstart_q, seqstart_k, num_seqs, total_q, total_k, max_seqlen_q,
                    max_seqlen_k, Hq, Hkv, D, dtype, causal, alibi_slopes, scale, stream) -> int:
    return load().mea_fwd_noalloc(q, k, v, out, lse, seqstart_q, seqstart_k, num_seqs, total_q, total_k,
                                  max_seqlen_q, max_seqlen_k, Hq, Hkv, D, dtype, causal, alibi_slopes,
                                  scale, stream)


def mea_fwd_splitkv(q, k, v, out, lse, seqstart_q, seqstart_k, num_seqs, total_q, total_k,
                    max_seqlen_q, max_seqlen_k, Hq, Hkv, D, dtype, causal, alibi_slopes, scale,
                    workspace, workspace_bytes, stream, chunk_keys) -> int:
    return load().mea_fwd_splitkv(q, k, v, out, lse, seqstart_q, seqstart_k, num_seqs, total_q,
                                  total_k, max_seqlen_q, max_seqlen_k, Hq, Hkv, D, dtype, causal,
                                  alibi_slopes, scale, workspace, workspace_bytes, stream,
                                  chunk_keys)


def mea_fwd_paged(q, k_cache, v_cache, out, lse, seqstart_q, seqstart_k, block_table, num_seqs,
                  total_q, total_k, max_seqlen_q, max_seqlen_k, page_size, num_pages, max_blocks, Hq,
                  Hkv, D, dtype, causal, alibi_slopes, scale, workspace, workspace_bytes, stream) -> int:
    return load().mea_fwd_paged(q, k_cache, v_cache, out, lse, seqstart_q, seqstart_k, block_table,
                                num_seqs, total_q, total_k, max_seqlen_q, max_seqlen_k, page_size,
                                num_pages, max_blocks, Hq, Hkv, D, dtype, causal, alibi_slopes, scale,
                                workspace, workspace_bytes, stream)


def mea_fwd_workspace_size(num_seqs, total_k, max_seqlen_q, max_seqlen_k, Hq, Hkv, D,
                           chunk_keys=0) -> int:
    return int(load().mea_fwd_workspace_size(num_seqs, total_k, max_seqlen_q, max_seqlen_k, Hq,
                                             Hkv, D, chunk_keys))


def mea_default_chunk_keys(total_k, Hq, Hkv) -> int:
    return int(load().mea_default_chunk_keys(total_k, Hq, Hkv))


def mea_bwd(q, k, v, out, lse, dout, dq, dk, dv, seqstart_q, seqstart_k, num_seqs, total_q, total_k,
            max_seqlen_q, max_seqlen_k, Hq, Hkv, D, dtype, causal, alibi_slopes, scale, workspace,
            workspace_bytes, stream) -> int:
    return load().mea_bwd(q, k, v, out, lse, dout, dq, dk, dv, seqstart_q, seqstart_k, num_seqs,
                          total_q, total_k, max_seqlen_q, max_seqlen_k, Hq, Hkv, D, dtype, causal,
                          alibi_slopes, scale, workspace, workspace_bytes, stream)


def mea_bwd_workspace_size(num_seqs, total_q, total_k, Hq, Hkv, D) -> int:
    return int(load().mea_bwd_workspace_size(num_seqs, total_q, total_k, Hq, Hkv, D))


def mea_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, out, lse, seqstart_q, seqstart_k, num_seqs, total_q,
                total_k, max_seqlen_q, max_seqlen_k, Hq, Hkv, D, out_dtype, causal, alibi_slopes, scale,
                workspace, workspace_bytes, stream) -> int:
    return load().mea_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, out, lse, seqstart_q, seqstart_k, num_seqs,
                              total_q, total_k, max_seqlen_q, max_seqlen_k, Hq, Hkv, D, out_dtype, causal,
                              alibi_slopes, scale, workspace, workspace_bytes, stream)


def mea_fwd_paged_fp8(q, k_cache, v_cache, q_scale, k_scale, v_scale, out, lse, seqstart_q, seqstart_k,
                      block_table, num_seqs, total_q, total_k, max_seqlen_q, max_seqlen_k, page_size, num_pages,
                      max_blocks, Hq, Hkv, D, out_dtype, causal, alibi_slopes, scale, workspace, workspace_bytes,
                      stream) -> int:
    return load().mea_fwd_paged_fp8(q, k_cache, v_cache, q_scale, k_scale, v_scale, out, lse, seqstart_q,
                                    seqstart_k, block_table, num_seqs, total_q, total_k, max_seqlen_q,
                                    max_seqlen_k, page_size, num_pages, max_blocks, Hq, Hkv, D, out_dtype, causal,
                                    alibi_slopes, scale, workspace, workspace_bytes, stream)


def mea_fwd_fp8_workspace_size(num_seqs, total_k, max_seqlen_q, max_seqlen_k, Hq, Hkv, D) -> int:
    return int(load().mea_fwd_fp8_workspace_size(num_seqs, total_k, max_seqlen_q, max_seqlen_k, Hq, Hkv, D))


def mea_swiglu_ffn(x, w_gate, w_up, w_down, hidden, out, tokens, d_model, d_ff, dtype, stream) -> int:
    return load().mea_swiglu_ffn(x, w_gate, w_up, w_down, hidden, out, tokens, d_model, d_ff, dtype, stream)


def mea_status_string(status: int) -> str:
    return load().mea_status_string(status).decode()


def mea_last_error() -> str:
    return load().mea_last_error().decode()


def mea_abi_version() -> int:
    return int(load().mea_abi_version())
