"""Python front end: xFormers-style masks and the attention call.

Marshalling only: shapes are checked and viewed packed, outputs and the
decode workspace are allocated with torch (device memory and streams are all
torch provides here), and every step of the computation runs in the HIP
library through ``_native``.  The call surface follows the tutorial page
"Cómo construir transformadores con memoria eficiente con xFormers ..."
(7minutos.es): section 4 (``BlockDiagonalMask.from_seqlens``, the causal
variant, ``memory_efficient_attention(q, k, v, attn_bias=...)`` on a packed
``[1, total, H, K]`` batch, and ``mask.split(out)``), and section 5 (the
5-D BMGHK grouped-query layout ``[B, M, G, Hq, K]`` with key/value heads
``[B, M, G, 1, K]``).
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple, Union

import numpy as np
import torch

from . import _native

__all__ = [
    "BlockDiagonalMask", "BlockDiagonalCausalMask", "memory_efficient_attention",
    "attention_packed", "attention_paged", "attention_backward_packed", "attention_packed_fp8",
    "attention_paged_fp8", "swiglu_ffn", "MeaError",
]


class MeaError(RuntimeError):
    """A non-OK status from the C entry point (its code is ``.status``)."""

    def __init__(self, status: int, detail: str):
        super().__init__(f"{_native.mea_status_string(status)}: {detail}")
        self.status = status


def _seqstart(lengths: Sequence[int]) -> List[int]:
    out = [0]
    for L in lengths:
        out.append(out[-1] + int(L))
    return out


class BlockDiagonalMask:
    """Attention only within each packed sequence (no padding between them).

    ``q_seqlen[b]`` queries of sequence b attend to its ``kv_seqlen[b]``
    keys; both are packed back to back along the token axis.
    """

    causal = False

    def __init__(self, q_seqlen: Sequence[int], kv_seqlen: Optional[Sequence[int]] = None):
        q = [int(x) for x in q_seqlen]
        kv = list(q) if kv_seqlen is None else [int(x) for x in kv_seqlen]
        if len(q) != len(kv):
            raise ValueError(f"{len(q)} query lengths but {len(kv)} key lengths")
        if any(x < 0 for x in q) or any(x < 0 for x in kv):
            raise ValueError("sequence lengths must be non-negative")
        self.q_seqlen: List[int] = q
        self.kv_seqlen: List[int] = kv
        self.q_seqstart: List[int] = _seqstart(q)
        self.kv_seqstart: List[int] = _seqstart(kv)
        self._dev = {}

    @classmethod
    def from_seqlens(cls, q_seqlen: Sequence[int], kv_seqlen: Optional[Sequence[int]] = None):
        return cls(q_seqlen, kv_seqlen)

    @property
    def num_seqs(self) -> int:
        return len(self.q_seqlen)

    @property
    def total_q(self) -> int:
        return self.q_seqstart[-1]

    @property
    def total_kv(self) -> int:
        return self.kv_seqstart[-1]

    @property
    def max_seqlen_q(self) -> int:
        return max(self.q_seqlen, default=0)

    @property
    def max_seqlen_kv(self) -> int:
        return max(self.kv_seqlen, default=0)

    def mixed_split(self) -> Optional[Tuple[int, int, int, int]]:
        """For a batch of prefills followed by decode steps (one query each),
        the way a serving engine lays out a mixed batch, ``(num_prefill_seqs,
        prefill_total_q, prefill_total_k, decode_max_seqlen_k)``; None when the
        batch has no such tail of decode steps or no prefill before it."""
        n = self.num_seqs
        i = n
        while i > 0 and self.q_seqlen[i - 1] == 1:
            i -= 1
        if i == n or max(self.q_seqlen[:i], default=0) <= 1:
            return None
        return i, self.q_seqstart[i], self.kv_seqstart[i], max(self.kv_seqlen[i:])

    def seqstart_tensors(self, device) -> Tuple[torch.Tensor, torch.Tensor]:
        """int32 device copies of the sequence offsets (cached per device)."""
        key = str(torch.device(device))
        if key not in self._dev:
            self._dev[key] = (torch.tensor(self.q_seqstart, dtype=torch.int32, device=device),
                              torch.tensor(self.kv_seqstart, dtype=torch.int32, device=device))
        return self._dev[key]

    def split(self, x: torch.Tensor) -> List[torch.Tensor]:
        """Per-sequence views of a packed query-side tensor ``[1, total_q, ...]``
        (or ``[total_q, ...]``): piece b is ``[1, q_seqlen[b], ...]``."""
        return self._split(x, self.q_seqstart)

    def split_kv(self, x: torch.Tensor) -> List[torch.Tensor]:
        return self._split(x, self.kv_seqstart)

    @staticmethod
    def _split(x: torch.Tensor, starts: List[int]) -> List[torch.Tensor]:
        packed = x[0] if (x.dim() >= 2 and x.shape[0] == 1 and x.shape[1] == starts[-1]) else x
        if packed.shape[0] != starts[-1]:
            raise ValueError(f"tensor has {packed.shape[0]} rows, mask covers {starts[-1]}")
        return [packed[starts[b]:starts[b + 1]].unsqueeze(0) for b in range(len(starts) - 1)]


class BlockDiagonalCausalMask(BlockDiagonalMask):
    """Block-diagonal plus a causal mask inside each sequence.  When a
    sequence has fewer queries than keys, its queries are its last positions."""

    causal = True


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float16:
        return _native.MEA_F16
    if dt == torch.bfloat16:
        return _native.MEA_BF16
    raise TypeError(f"dtype {dt} is not supported (float16 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_out(t: Optional[torch.Tensor], name: str, shape, dtype: torch.dtype, dev: torch.device) -> None:
    """A caller-supplied output buffer must be exactly what the kernels write:
    the kernels store full-size rows through its raw pointer, so a short,
    strided, wrongly typed or foreign-device buffer would be written out of
    bounds or scrambled."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != dev:
        raise ValueError(f"{name} must be on {dev}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(ws: Optional[torch.Tensor], need: int, dev: torch.device) -> Optional[torch.Tensor]:
    """The caller's workspace if it is a usable one of at least ``need`` bytes,
    else a new one (``None`` when nothing is needed)."""
    if need <= 0:
        return None
    if ws is not None:
        if ws.device != dev:
            raise ValueError(f"workspace must be on {dev}, got {ws.device}")
        if not ws.is_contiguous():
            raise ValueError("workspace must be contiguous")
        if ws.numel() * ws.element_size() >= need:
            return ws
    return torch.empty(need, dtype=torch.uint8, device=dev)


def attention_packed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     seqstart_q: torch.Tensor, seqstart_k: torch.Tensor,
                     max_seqlen_q: int, max_seqlen_k: int, *, causal: bool = False,
                     alibi_slopes: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                     return_lse: bool = False, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     chunk_keys: Optional[int] = None, mixed: Optional[Tuple[int, int, int, int]] = None,
                     stream: Optional[torch.cuda.Stream] = None):
    """Packed call: q ``[Tq, Hq, D]``, k/v ``[Tk, Hkv, D]`` (contiguous device
    tensors), int32 device ``seqstart_q/k`` ``[n + 1]``.  Returns ``out`` or
    ``(out, lse)`` with lse ``[Hq, Tq]`` float32.  ``chunk_keys`` forces the
    decode split length (only for max_seqlen_q == 1).  ``mixed`` =
    ``(num_prefill_seqs, prefill_total_q, prefill_total_k,
    decode_max_seqlen_k)`` serves a batch of prefills followed by one-query
    decode steps with both kinds of kernels (mea_fwd_mixed; see
    ``BlockDiagonalMask.mixed_split``)."""
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("packed q, k, v must be [tokens, heads, D]")
    Tq, Hq, D = q.shape
    Tk, Hkv, Dk = k.shape
    if Dk != D or tuple(v.shape) != (Tk, Hkv, D):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    dev = q.device
    if dev.type != "cuda" or k.device != dev or v.device != dev:
        raise ValueError("q, k and v must be on the same GPU")
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    if seqstart_q.dtype != torch.int32 or seqstart_k.dtype != torch.int32:
        raise TypeError("seqstart tensors must be int32")
    if seqstart_q.device != dev or seqstart_k.device != dev:
        raise ValueError("seqstart tensors must be on the same GPU as q")
    num_seqs = seqstart_q.numel() - 1
    if seqstart_k.numel() != num_seqs + 1:
        raise ValueError("seqstart_q and seqstart_k differ in length")
    _check_out(out, "out", (Tq, Hq, D), q.dtype, dev)
    _check_out(lse, "lse", (Hq, Tq), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=dev)
    slopes = None
    if alibi_slopes is not None:
        slopes = alibi_slopes.to(device=dev, dtype=torch.float32).contiguous()
        if slopes.numel() != Hq:
            raise ValueError(f"alibi_slopes needs {Hq} values (one per query head)")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    scale = float(np.float32(scale))
    if mixed is not None:
        if chunk_keys is not None:
            raise ValueError("chunk_keys and mixed are exclusive")
        n_pre, pre_q, pre_k, dec_max_k = (int(x) for x in mixed)
        ws_bytes = _native.mea_fwd_mixed_workspace_size(num_seqs, Tk, int(max_seqlen_q), int(max_seqlen_k), n_pre,
                                                        pre_k, dec_max_k, Hq, Hkv, D)
    else:
        ws_bytes = _native.mea_fwd_workspace_size(num_seqs, Tk, max_seqlen_q, max_seqlen_k, Hq, Hkv, D,
                                                  int(chunk_keys or 0))
    workspace = _workspace(workspace, ws_bytes, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(seqstart_q), _ptr(seqstart_k),
            num_seqs, Tq, Tk, int(max_seqlen_q), int(max_seqlen_k))
    tail = (Hq, Hkv, D, _dtype_code(q.dtype), int(bool(causal)), _ptr(slopes), scale, _ptr(workspace),
            ws_bytes, stream.cuda_stream)
    with torch.cuda.device(dev):
        if mixed is not None:
            st = _native.mea_fwd_mixed(*head, n_pre, pre_q, pre_k, dec_max_k, *tail)
        elif chunk_keys is None:
            st = _native.mea_fwd(*head, *tail)
        else:
            st = _native.mea_fwd_splitkv(*head, *tail, int(chunk_keys))
    if st != _native.MEA_OK:
        raise MeaError(st, _native.mea_last_error())
    return (out, lse) if return_lse else out


def attention_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    block_table: torch.Tensor, seqstart_q: torch.Tensor, seqstart_k: torch.Tensor,
                    max_seqlen_q: int, max_seqlen_k: int, *, causal: bool = False,
                    alibi_slopes: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                    return_lse: bool = False, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    total_k: Optional[int] = None, stream: Optional[torch.cuda.Stream] = None):
    """Packed queries over a paged K/V cache: q ``[Tq, Hq, D]``, k/v cache
    ``[num_pages, page_size, Hkv, D]``, int32 device ``block_table``
    ``[n, max_blocks]`` (page of each page_size-key block of a sequence) and
    int32 device ``seqstart_q/k`` ``[n + 1]`` (logical key offsets).
    ``total_k`` is the total number of keys (read from ``seqstart_k``, with a
    device synchronisation, when not given).  Returns ``out`` or
    ``(out, lse)`` as :func:`attention_packed` does."""
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("q must be [tokens, heads, D] and the caches [pages, page_size, heads, D]")
    Tq, Hq, D = q.shape
    num_pages, page_size, Hkv, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k_cache {tuple(k_cache.shape)} "
                         f"v_cache {tuple(v_cache.shape)}")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q and the caches must share a dtype")
    dev = q.device
    if dev.type != "cuda" or k_cache.device != dev or v_cache.device != dev or block_table.device != dev:
        raise ValueError("q, the caches and block_table must be on the same GPU")
    if block_table.dtype != torch.int32 or block_table.dim() != 2:
        raise TypeError("block_table must be an int32 [num_seqs, max_blocks] tensor")
    q, k_cache, v_cache = q.contiguous(), k_cache.contiguous(), v_cache.contiguous()
    block_table = block_table.contiguous()
    if seqstart_q.dtype != torch.int32 or seqstart_k.dtype != torch.int32:
        raise TypeError("seqstart tensors must be int32")
    num_seqs = seqstart_q.numel() - 1
    if seqstart_k.numel() != num_seqs + 1 or block_table.shape[0] != num_seqs:
        raise ValueError("seqstart_q, seqstart_k and block_table disagree on the number of sequences")
    Tk = int(total_k) if total_k is not None else (int(seqstart_k[-1].item()) if num_seqs > 0 else 0)
    _check_out(out, "out", (Tq, Hq, D), q.dtype, dev)
    _check_out(lse, "lse", (Hq, Tq), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=dev)
    slopes = None
    if alibi_slopes is not None:
        slopes = alibi_slopes.to(device=dev, dtype=torch.float32).contiguous()
        if slopes.numel() != Hq:
            raise ValueError(f"alibi_slopes needs {Hq} values (one per query head)")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    scale = float(np.float32(scale))
    ws_bytes = _native.mea_fwd_workspace_size(num_seqs, Tk, max_seqlen_q, max_seqlen_k, Hq, Hkv, D, 0)
    workspace = _workspace(workspace, ws_bytes, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = _native.mea_fwd_paged(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), _ptr(seqstart_q),
            _ptr(seqstart_k), _ptr(block_table), num_seqs, Tq, Tk, int(max_seqlen_q), int(max_seqlen_k),
            page_size, num_pages, block_table.shape[1], Hq, Hkv, D, _dtype_code(q.dtype),
            int(bool(causal)), _ptr(slopes), scale, _ptr(workspace),
            ws_bytes, stream.cuda_stream)
    if st != _native.MEA_OK:
        raise MeaError(st, _native.mea_last_error())
    return (out, lse) if return_lse else out


def attention_backward_packed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                              lse: torch.Tensor, dout: torch.Tensor, seqstart_q: torch.Tensor,
                              seqstart_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, *,
                              causal: bool = False, alibi_slopes: Optional[torch.Tensor] = None,
                              scale: Optional[float] = None, dq: Optional[torch.Tensor] = None,
                              dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
                              workspace: Optional[torch.Tensor] = None,
                              stream: Optional[torch.cuda.Stream] = None):
    """Gradients of the packed attention: the arguments of the forward call
    (q, k, v, offsets, masks, slopes, scale), its ``out`` and ``lse``, and the
    upstream gradient ``dout`` (shaped like ``out``).  Returns ``(dq, dk, dv)``
    shaped like q, k and v."""
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("packed q, k, v must be [tokens, heads, D]")
    Tq, Hq, D = q.shape
    Tk, Hkv, Dk = k.shape
    if Dk != D or tuple(v.shape) != (Tk, Hkv, D):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if tuple(out.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("out and dout must be shaped like q")
    if tuple(lse.shape) != (Hq, Tq) or lse.dtype != torch.float32:
        raise ValueError(f"lse must be float32 [{Hq}, {Tq}]")
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype):
        raise TypeError("q, k, v, out and dout must share a dtype")
    dev = q.device
    if dev.type != "cuda" or any(t.device != dev for t in (k, v, out, lse, dout, seqstart_q, seqstart_k)):
        raise ValueError("all tensors must be on the same GPU")
    q, k, v, out, lse, dout = (t.contiguous() for t in (q, k, v, out, lse, dout))
    if seqstart_q.dtype != torch.int32 or seqstart_k.dtype != torch.int32:
        raise TypeError("seqstart tensors must be int32")
    num_seqs = seqstart_q.numel() - 1
    if seqstart_k.numel() != num_seqs + 1:
        raise ValueError("seqstart_q and seqstart_k differ in length")
    _check_out(dq, "dq", q.shape, q.dtype, dev)
    _check_out(dk, "dk", k.shape, k.dtype, dev)
    _check_out(dv, "dv", v.shape, v.dtype, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    slopes = None
    if alibi_slopes is not None:
        slopes = alibi_slopes.to(device=dev, dtype=torch.float32).contiguous()
        if slopes.numel() != Hq:
            raise ValueError(f"alibi_slopes needs {Hq} values (one per query head)")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    scale = float(np.float32(scale))
    ws_bytes = _native.mea_bwd_workspace_size(num_seqs, Tq, Tk, Hq, Hkv, D)
    workspace = _workspace(workspace, ws_bytes, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = _native.mea_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(seqstart_q), _ptr(seqstart_k), num_seqs, Tq, Tk, int(max_seqlen_q), int(max_seqlen_k),
            Hq, Hkv, D, _dtype_code(q.dtype), int(bool(causal)), _ptr(slopes), scale,
            _ptr(workspace), ws_bytes, stream.cuda_stream)
    if st != _native.MEA_OK:
        raise MeaError(st, _native.mea_last_error())
    return dq, dk, dv


class _PackedAttention(torch.autograd.Function):
    """Autograd node of the packed attention: forward through ``mea_fwd``
    (keeping out and lse), backward through ``mea_bwd``."""

    @staticmethod
    def forward(ctx, q, k, v, seqstart_q, seqstart_k, max_seqlen_q, max_seqlen_k, causal, slopes, scale, mixed):
        out, lse = attention_packed(q, k, v, seqstart_q, seqstart_k, max_seqlen_q, max_seqlen_k,
                                    causal=causal, alibi_slopes=slopes, scale=scale, return_lse=True, mixed=mixed)
        ctx.save_for_backward(q, k, v, out, lse, seqstart_q, seqstart_k)
        ctx.meta = (max_seqlen_q, max_seqlen_k, causal, slopes, scale)
        ctx.mark_non_differentiable(lse)
        return out, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        q, k, v, out, lse, seqstart_q, seqstart_k = ctx.saved_tensors
        max_seqlen_q, max_seqlen_k, causal, slopes, scale = ctx.meta
        dq, dk, dv = attention_backward_packed(q, k, v, out, lse, dout.contiguous(), seqstart_q, seqstart_k,
                                               max_seqlen_q, max_seqlen_k, causal=causal,
                                               alibi_slopes=slopes, scale=scale)
        return dq, dk, dv, None, None, None, None, None, None, None, None


def attention_packed_fp8(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, q_scale: float,
                         k_scale: float, v_scale: float, seqstart_q: torch.Tensor, seqstart_k: torch.Tensor,
                         max_seqlen_q: int, max_seqlen_k: int, *, causal: bool = False,
                         alibi_slopes: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                         out_dtype: torch.dtype = torch.bfloat16, return_lse: bool = False,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None,
                         stream: Optional[torch.cuda.Stream] = None):
    """Packed call on 8-bit inputs: ``q8 [Tq, Hq, 128]``, ``k8``/``v8``
    ``[Tk, Hkv, 128]`` of ``torch.float8_e4m3fn`` with one scale per tensor
    (the values are scale * tensor).  Returns ``out`` of ``out_dtype`` (or
    ``(out, lse)``), as :func:`attention_packed` does on the dequantised
    values."""
    if q8.dim() != 3 or k8.dim() != 3 or v8.dim() != 3:
        raise ValueError("packed q8, k8, v8 must be [tokens, heads, D]")
    Tq, Hq, D = q8.shape
    Tk, Hkv, Dk = k8.shape
    if Dk != D or tuple(v8.shape) != (Tk, Hkv, D):
        raise ValueError(f"shape mismatch: q8 {tuple(q8.shape)} k8 {tuple(k8.shape)} v8 {tuple(v8.shape)}")
    if not (q8.dtype == k8.dtype == v8.dtype == torch.float8_e4m3fn):
        raise TypeError("q8, k8 and v8 must be torch.float8_e4m3fn")
    dev = q8.device
    if dev.type != "cuda" or k8.device != dev or v8.device != dev:
        raise ValueError("q8, k8 and v8 must be on the same GPU")
    q8, k8, v8 = q8.contiguous(), k8.contiguous(), v8.contiguous()
    if seqstart_q.dtype != torch.int32 or seqstart_k.dtype != torch.int32:
        raise TypeError("seqstart tensors must be int32")
    num_seqs = seqstart_q.numel() - 1
    if seqstart_k.numel() != num_seqs + 1:
        raise ValueError("seqstart_q and seqstart_k differ in length")
    _check_out(out, "out", (Tq, Hq, D), out_dtype, dev)
    _check_out(lse, "lse", (Hq, Tq), torch.float32, dev)
    if out is None:
        out = torch.empty((Tq, Hq, D), dtype=out_dtype, device=dev)
    if return_lse and lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=dev)
    slopes = None
    if alibi_slopes is not None:
        slopes = alibi_slopes.to(device=dev, dtype=torch.float32).contiguous()
        if slopes.numel() != Hq:
            raise ValueError(f"alibi_slopes needs {Hq} values (one per query head)")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    scale = float(np.float32(scale))
    ws_bytes = _native.mea_fwd_fp8_workspace_size(num_seqs, Tk, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, D)
    workspace = _workspace(workspace, ws_bytes, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = _native.mea_fwd_fp8(
            _ptr(q8), _ptr(k8), _ptr(v8), float(q_scale), float(k_scale), float(v_scale), _ptr(out), _ptr(lse),
            _ptr(seqstart_q), _ptr(seqstart_k), num_seqs, Tq, Tk, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv,
            D, _dtype_code(out.dtype), int(bool(causal)), _ptr(slopes), scale,
            _ptr(workspace), ws_bytes, stream.cuda_stream)
    if st != _native.MEA_OK:
        raise MeaError(st, _native.mea_last_error())
    return (out, lse) if return_lse else out


def attention_paged_fp8(q8: torch.Tensor, k_cache8: torch.Tensor, v_cache8: torch.Tensor, q_scale: float,
                        k_scale: float, v_scale: float, block_table: torch.Tensor, seqstart_q: torch.Tensor,
                        seqstart_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, *, causal: bool = False,
                        alibi_slopes: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                        out_dtype: torch.dtype = torch.bfloat16, return_lse: bool = False,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, total_k: Optional[int] = None,
                        stream: Optional[torch.cuda.Stream] = None):
    """:func:`attention_packed_fp8` over a paged fp8 K/V cache: q8
    ``[Tq, Hq, 128]`` and caches ``[num_pages, page_size, Hkv, 128]`` of
    ``torch.float8_e4m3fn``, the ``block_table`` and ``seqstart`` arrays and
    ``total_k`` as for :func:`attention_paged`."""
    if q8.dim() != 3 or k_cache8.dim() != 4 or v_cache8.dim() != 4:
        raise ValueError("q8 must be [tokens, heads, D] and the caches [pages, page_size, heads, D]")
    Tq, Hq, D = q8.shape
    num_pages, page_size, Hkv, Dk = k_cache8.shape
    if Dk != D or tuple(v_cache8.shape) != tuple(k_cache8.shape):
        raise ValueError(f"shape mismatch: q8 {tuple(q8.shape)} k_cache8 {tuple(k_cache8.shape)} "
                         f"v_cache8 {tuple(v_cache8.shape)}")
    if not (q8.dtype == k_cache8.dtype == v_cache8.dtype == torch.float8_e4m3fn):
        raise TypeError("q8 and the caches must be torch.float8_e4m3fn")
    dev = q8.device
    if dev.type != "cuda" or k_cache8.device != dev or v_cache8.device != dev or block_table.device != dev:
        raise ValueError("q8, the caches and block_table must be on the same GPU")
    if block_table.dtype != torch.int32 or block_table.dim() != 2:
        raise TypeError("block_table must be an int32 [num_seqs, max_blocks] tensor")
    q8, k_cache8, v_cache8 = q8.contiguous(), k_cache8.contiguous(), v_cache8.contiguous()
    block_table = block_table.contiguous()
    if seqstart_q.dtype != torch.int32 or seqstart_k.dtype != torch.int32:
        raise TypeError("seqstart tensors must be int32")
    num_seqs = seqstart_q.numel() - 1
    if seqstart_k.numel() != num_seqs + 1 or block_table.shape[0] != num_seqs:
        raise ValueError("seqstart_q, seqstart_k and block_table disagree on the number of sequences")
    Tk = int(total_k) if total_k is not None else (int(seqstart_k[-1].item()) if num_seqs > 0 else 0)
    _check_out(out, "out", (Tq, Hq, D), out_dtype, dev)
    _check_out(lse, "lse", (Hq, Tq), torch.float32, dev)
    if out is None:
        out = torch.empty((Tq, Hq, D), dtype=out_dtype, device=dev)
    if return_lse and lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=dev)
    slopes = None
    if alibi_slopes is not None:
        slopes = alibi_slopes.to(device=dev, dtype=torch.float32).contiguous()
        if slopes.numel() != Hq:
            raise ValueError(f"alibi_slopes needs {Hq} values (one per query head)")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    scale = float(np.float32(scale))
    ws_bytes = _native.mea_fwd_fp8_workspace_size(num_seqs, Tk, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, D)
    workspace = _workspace(workspace, ws_bytes, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = _native.mea_fwd_paged_fp8(
            _ptr(q8), _ptr(k_cache8), _ptr(v_cache8), float(q_scale), float(k_scale), float(v_scale), _ptr(out),
            _ptr(lse), _ptr(seqstart_q), _ptr(seqstart_k), _ptr(block_table), num_seqs, Tq, Tk,
            int(max_seqlen_q), int(max_seqlen_k), page_size, num_pages, block_table.shape[1], Hq, Hkv, D,
            _dtype_code(out.dtype), int(bool(causal)), _ptr(slopes), scale,
            _ptr(workspace), ws_bytes, stream.cuda_stream)
    if st != _native.MEA_OK:
        raise MeaError(st, _native.mea_last_error())
    return (out, lse) if return_lse else out


def swiglu_ffn(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor, *,
               hidden: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
               return_hidden: bool = False, stream: Optional[torch.cuda.Stream] = None):
    """SwiGLU feed-forward: ``(SiLU(x w_gate^T) * (x w_up^T)) w_down^T`` for
    ``x [tokens, d_model]``, ``w_gate``/``w_up [d_ff, d_model]``,
    ``w_down [d_model, d_ff]`` (torch Linear weight layout).  Returns ``out``
    (and the hidden activations if ``return_hidden``)."""
    if x.dim() != 2:
        raise ValueError("x must be [tokens, d_model]")
    T, d_model = x.shape
    d_ff = w_gate.shape[0]
    if tuple(w_gate.shape) != (d_ff, d_model) or tuple(w_up.shape) != (d_ff, d_model) \
            or tuple(w_down.shape) != (d_model, d_ff):
        raise ValueError(f"weight shapes {tuple(w_gate.shape)}, {tuple(w_up.shape)}, {tuple(w_down.shape)} "
                         f"do not match x {tuple(x.shape)}")
    if not (x.dtype == w_gate.dtype == w_up.dtype == w_down.dtype):
        raise TypeError("x and the weights must share a dtype")
    dev = x.device
    if dev.type != "cuda" or any(t.device != dev for t in (w_gate, w_up, w_down)):
        raise ValueError("x and the weights must be on the same GPU")
    x, w_gate, w_up, w_down = (t.contiguous() for t in (x, w_gate, w_up, w_down))
    _check_out(hidden, "hidden", (T, d_ff), x.dtype, dev)
    _check_out(out, "out", (T, d_model), x.dtype, dev)
    if hidden is None:
        hidden = torch.empty((T, d_ff), dtype=x.dtype, device=dev)
    if out is None:
        out = torch.empty((T, d_model), dtype=x.dtype, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = _native.mea_swiglu_ffn(_ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(hidden), _ptr(out), T,
                                    d_model, d_ff, _dtype_code(x.dtype), stream.cuda_stream)
    if st != _native.MEA_OK:
        raise MeaError(st, _native.mea_last_error())
    return (out, hidden) if return_hidden else out


def _kv_heads_bmghk(k: torch.Tensor, hq: int) -> torch.Tensor:
    """[B, M, G, Hk, K] key/value tensor with Hk == 1 (or broadcast along that
    axis) -> [B, M, G, K]; Hk == hq (one K/V head per query head) -> [B, M, G*hq, K]."""
    B, M, G, Hk, K = k.shape
    if Hk == 1 or k.stride(3) == 0:
        return k[:, :, :, 0, :]
    if Hk == hq:
        return k.reshape(B, M, G * Hk, K)
    raise ValueError(f"BMGHK key/value head axis must be 1 or {hq}, got {Hk}")


def memory_efficient_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                               attn_bias: Optional[BlockDiagonalMask] = None, *,
                               scale: Optional[float] = None,
                               alibi_slopes: Optional[torch.Tensor] = None,
                               return_lse: bool = False):
    """softmax(q k^T * scale + bias) v without materialising the scores.

    Layouts: BMHK ``q [B, M, Hq, K]``, ``k/v [B, Mk, Hkv, K]`` with Hq a
    multiple of Hkv (query head h reads key/value head h // (Hq/Hkv)); or BMGHK
    ``q [B, M, G, Hq, K]``, ``k/v [B, Mk, G, 1, K]`` (G groups).  Without a
    mask every batch element is attended on its own; with a
    ``BlockDiagonalMask`` / ``BlockDiagonalCausalMask`` the batch must be 1
    and the token axis is the packed sequences.  ``alibi_slopes`` (one per
    query head, in the flattened head order) adds -slope * |i - j| with
    sequence-local positions.  Returns a tensor shaped like ``q`` (and the
    log-sum-exp ``[Hq_total, B*M]`` float32 if ``return_lse``).  Differentiable
    in q, k and v: when any of them requires grad, the backward runs the HIP
    backward kernels (``mea_bwd``).
    """
    if q.dim() == 5:
        B, M, G, Hg, K = q.shape
        qp = q.reshape(B * M, G * Hg, K)
        kp = _kv_heads_bmghk(k, Hg)
        vp = _kv_heads_bmghk(v, Hg)
        Mk = kp.shape[1]
        kp = kp.reshape(B * Mk, kp.shape[2], K)
        vp = vp.reshape(B * Mk, vp.shape[2], K)
    elif q.dim() == 4:
        B, M, Hq, K = q.shape
        Mk = k.shape[1]
        qp = q.reshape(B * M, Hq, K)
        kp = k.reshape(B * Mk, k.shape[2], K)
        vp = v.reshape(B * Mk, v.shape[2], K)
    else:
        raise ValueError("q must be BMHK [B, M, H, K] or BMGHK [B, M, G, H, K]")
    if tuple(k.shape) != tuple(v.shape):
        raise ValueError("k and v must have the same shape")
    if attn_bias is None:
        mask = BlockDiagonalMask([M] * B, [Mk] * B)
    else:
        if not isinstance(attn_bias, BlockDiagonalMask):
            raise TypeError(f"unsupported attn_bias {type(attn_bias).__name__}")
        if B != 1:
            raise ValueError("a block-diagonal mask needs batch size 1 (sequences packed along M)")
        if attn_bias.total_q != M or attn_bias.total_kv != Mk:
            raise ValueError(f"mask covers {attn_bias.total_q} queries / {attn_bias.total_kv} keys, "
                             f"tensors have {M} / {Mk}")
        mask = attn_bias
    ssq, ssk = mask.seqstart_tensors(q.device)
    if torch.is_grad_enabled() and (q.requires_grad or k.requires_grad or v.requires_grad):
        out, lse = _PackedAttention.apply(qp.contiguous(), kp.contiguous(), vp.contiguous(), ssq, ssk,
                                          mask.max_seqlen_q, mask.max_seqlen_kv, mask.causal,
                                          alibi_slopes, scale, mask.mixed_split())
        return (out.view(q.shape), lse) if return_lse else out.view(q.shape)
    res = attention_packed(qp, kp, vp, ssq, ssk, mask.max_seqlen_q, mask.max_seqlen_kv,
                           causal=mask.causal, alibi_slopes=alibi_slopes, scale=scale,
                           return_lse=return_lse, mixed=mask.mixed_split())
    if return_lse:
        return res[0].view(q.shape), res[1]
    return res.view(q.shape)
