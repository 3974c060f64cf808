"""Guard bytes around every buffer the kernels write: out, lse, dq/dk/dv, the
SwiGLU hidden and out, and the workspace (decode partials, V^T tile images and
their flags, backward row terms).  Each buffer is the middle of a larger
allocation whose 4 KiB before and after hold a seeded byte pattern; after the
call the pattern must be intact (nothing written past either end) and the
buffer itself, pre-filled with NaN bytes, must be fully overwritten (outputs)."""
import sys

import pytest
import torch

from memory_efficient_attention_amd import _native
from mea_workloads import random_case, random_dout, swiglu_case, to_fp8, to_paged

pytestmark = pytest.mark.gpu

GUARD = 4096


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


class Guarded:
    """A buffer of `shape` and `dtype` between two guard regions of GUARD bytes."""

    def __init__(self, shape, dtype, fill_nan=True, nbytes=None):
        n = nbytes if nbytes is not None else torch.empty(shape, dtype=dtype, device="meta").numel() * \
            torch.empty((), dtype=dtype).element_size()
        self.n = n
        g = torch.Generator().manual_seed(n % 9973)
        pattern = torch.randint(0, 256, (2 * GUARD,), generator=g, dtype=torch.uint8)
        self.pattern = pattern
        host = torch.empty(GUARD + n + GUARD, dtype=torch.uint8)
        host[:GUARD] = pattern[:GUARD]
        host[GUARD + n:] = pattern[GUARD:]
        host[GUARD:GUARD + n] = 0xFF if fill_nan else 0x5A
        self.buf = host.cuda()
        mid = self.buf[GUARD:GUARD + n]
        self.t = mid.view(dtype).view(shape) if nbytes is None else mid

    def check(self, what, written=True):
        torch.cuda.synchronize()
        host = self.buf.cpu()
        assert torch.equal(host[:GUARD], self.pattern[:GUARD]), f"{what}: bytes before the buffer were written"
        assert torch.equal(host[GUARD + self.n:], self.pattern[GUARD:]), f"{what}: bytes past the buffer were written"
        if written and self.t.dtype.is_floating_point:
            assert not torch.isnan(self.t.float()).any().item(), f"{what}: part of the buffer was not written"


def _fwd_guarded(inp, fn_name="packed", chunk_keys=None, page_size=64, fp8=False):
    from memory_efficient_attention_amd import (attention_packed, attention_packed_fp8, attention_paged,
                                                attention_paged_fp8)
    dev = "cuda"
    Tq, Hq, D = inp.q.shape
    Tk, Hkv, _ = inp.k.shape
    out_dtype = inp.q.dtype
    out = Guarded((Tq, Hq, D), out_dtype)
    lse = Guarded((Hq, Tq), torch.float32)
    mixed = None
    if fn_name == "mixed":
        from memory_efficient_attention_amd import BlockDiagonalMask
        mixed = BlockDiagonalMask.from_seqlens(inp.seqlens_q, inp.seqlens_k).mixed_split()
        ws_n = _native.mea_fwd_mixed_workspace_size(len(inp.seqlens_q), Tk, inp.max_seqlen_q, inp.max_seqlen_k,
                                                    mixed[0], mixed[2], mixed[3], Hq, Hkv, D)
    elif fp8:
        ws_n = _native.mea_fwd_fp8_workspace_size(len(inp.seqlens_q), Tk, inp.max_seqlen_q, inp.max_seqlen_k, Hq, Hkv, D)
    else:
        ws_n = _native.mea_fwd_workspace_size(len(inp.seqlens_q), Tk, inp.max_seqlen_q, inp.max_seqlen_k, Hq, Hkv, D,
                                              int(chunk_keys or 0))
    ws = Guarded(None, torch.uint8, fill_nan=False, nbytes=ws_n)
    slopes = None if inp.alibi_slopes is None else inp.alibi_slopes.to(dev)
    ssq, ssk = inp.seqstart_q.to(dev), inp.seqstart_k.to(dev)
    kw = dict(causal=inp.causal, alibi_slopes=slopes, scale=inp.scale, return_lse=True, out=out.t, lse=lse.t,
              workspace=ws.t)
    if fp8:
        f8 = to_fp8(inp)
        if fn_name == "packed":
            attention_packed_fp8(f8.q8.to(dev), f8.k8.to(dev), f8.v8.to(dev), f8.q_scale, f8.k_scale, f8.v_scale,
                                 ssq, ssk, inp.max_seqlen_q, inp.max_seqlen_k, out_dtype=out_dtype, **kw)
        else:
            import dataclasses
            pk = to_paged(dataclasses.replace(inp, k=f8.k8, v=f8.v8), page_size, seed=1)
            attention_paged_fp8(f8.q8.to(dev), pk.k_cache.to(dev), pk.v_cache.to(dev), f8.q_scale, f8.k_scale,
                                f8.v_scale, pk.block_table.to(dev), ssq, ssk, inp.max_seqlen_q, inp.max_seqlen_k,
                                out_dtype=out_dtype, total_k=Tk, **kw)
    elif fn_name in ("packed", "mixed"):
        attention_packed(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), ssq, ssk, inp.max_seqlen_q, inp.max_seqlen_k,
                         chunk_keys=chunk_keys, mixed=mixed, **kw)
    else:
        pk = to_paged(inp, page_size, seed=1)
        attention_paged(inp.q.to(dev), pk.k_cache.to(dev), pk.v_cache.to(dev), pk.block_table.to(dev), ssq, ssk,
                        inp.max_seqlen_q, inp.max_seqlen_k, total_k=Tk, **kw)
    return out, lse, ws


FWD_CASES = [
    # (name, seqlens_q, seqlens_k, Hq, Hkv, D, dtype, causal, alibi, entry, chunk_keys, fp8)
    ("prefill_bf16_gqa", [130, 7, 200, 65], None, 8, 2, 128, "bf16", True, True, "packed", None, False),
    ("prefill_fp16_d64", [37, 120, 8, 200], None, 8, 8, 64, "fp16", False, False, "packed", None, False),
    ("decode_bf16", [1, 1, 1], [3000, 65, 1000], 16, 2, 128, "bf16", False, True, "packed", None, False),
    ("decode_split_64", [1, 1, 1], [3000, 65, 1000], 8, 8, 64, "fp16", False, False, "packed", 64, False),
    ("paged_prefill", [200, 17, 300], None, 12, 4, 128, "bf16", True, True, "paged", None, False),
    ("paged_decode", [1, 1, 1, 1], [1, 700, 129, 2000], 8, 2, 128, "bf16", False, False, "paged", None, False),
    ("fp8_prefill", [130, 7, 200], None, 8, 2, 128, "bf16", True, False, "packed", None, True),
    ("fp8_decode", [1, 1, 1], [3000, 65, 1000], 16, 8, 128, "bf16", False, False, "packed", None, True),
    ("fp8_paged_decode", [1, 1, 1], [3000, 65, 1000], 16, 8, 128, "bf16", False, False, "paged", None, True),
    ("mixed", [130, 7, 1, 1, 1], [130, 7, 3000, 65, 1000], 16, 2, 128, "bf16", True, True, "mixed", None, False),
]


@pytest.mark.parametrize("ci", range(len(FWD_CASES)))
def test_forward_writes_stay_in_bounds(ci):
    name, lq, lk, Hq, Hkv, D, dt, causal, alibi, entry, chunk, fp8 = FWD_CASES[ci]
    _log(f"canary {name}")
    inp = random_case(4300 + ci, lq, lk, Hq=Hq, Hkv=Hkv, D=D, dtype=dt, causal=causal, alibi=alibi)
    out, lse, ws = _fwd_guarded(inp, entry, chunk, fp8=fp8)
    out.check(f"{name} out")
    lse.check(f"{name} lse")
    ws.check(f"{name} workspace", written=False)


def test_backward_writes_stay_in_bounds():
    from memory_efficient_attention_amd import attention_backward_packed, attention_packed
    _log("canary backward")
    inp = random_case(4400, [130, 7, 200, 0, 65], [130, 7, 200, 40, 65], Hq=8, Hkv=2, D=128, dtype="bf16",
                      causal=True, alibi=True)
    dout = random_dout(4400, inp)
    dev = "cuda"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    ssq, ssk = inp.seqstart_q.to(dev), inp.seqstart_k.to(dev)
    slopes = inp.alibi_slopes.to(dev)
    o, l = attention_packed(q, k, v, ssq, ssk, inp.max_seqlen_q, inp.max_seqlen_k, causal=True, alibi_slopes=slopes,
                            scale=inp.scale, return_lse=True)
    dq, dk, dv = Guarded(q.shape, q.dtype), Guarded(k.shape, k.dtype), Guarded(v.shape, v.dtype)
    n = _native.mea_bwd_workspace_size(len(inp.seqlens_q), inp.total_q, inp.total_k, inp.Hq, inp.Hkv, inp.D)
    ws = Guarded(None, torch.uint8, fill_nan=False, nbytes=n)
    attention_backward_packed(q, k, v, o, l, dout.to(dev), ssq, ssk, inp.max_seqlen_q, inp.max_seqlen_k, causal=True,
                              alibi_slopes=slopes, scale=inp.scale, dq=dq.t, dk=dk.t, dv=dv.t, workspace=ws.t)
    for name, gbuf in (("dq", dq), ("dk", dk), ("dv", dv)):
        gbuf.check(f"backward {name}")
    ws.check("backward workspace", written=False)


def test_swiglu_writes_stay_in_bounds():
    from memory_efficient_attention_amd import swiglu_ffn
    _log("canary swiglu")
    f = swiglu_case(4500, 300, 256, 384, dtype="bf16")
    dev = "cuda"
    hidden = Guarded((300, 384), torch.bfloat16)
    out = Guarded((300, 256), torch.bfloat16)
    swiglu_ffn(f.x.to(dev), f.w_gate.to(dev), f.w_up.to(dev), f.w_down.to(dev), hidden=hidden.t, out=out.t)
    hidden.check("swiglu hidden")
    out.check("swiglu out")


def test_bad_output_buffers_raise():
    """The binding refuses an output buffer the kernels would write out of
    bounds or scramble (before any launch)."""
    from memory_efficient_attention_amd import attention_packed
    inp = random_case(4600, [64, 30], None, Hq=4, Hkv=2, D=64, dtype="bf16")
    dev = "cuda"
    args = (inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.seqstart_q.to(dev), inp.seqstart_k.to(dev),
            inp.max_seqlen_q, inp.max_seqlen_k)
    Tq, Hq, D = inp.q.shape
    bad_outs = [torch.empty((Tq - 1, Hq, D), dtype=torch.bfloat16, device=dev),
                torch.empty((Tq, Hq, D), dtype=torch.float32, device=dev),
                torch.empty((Hq, Tq, D), dtype=torch.bfloat16, device=dev).transpose(0, 1),
                torch.empty((Tq, Hq, D), dtype=torch.bfloat16)]
    for bad in bad_outs:
        with pytest.raises((ValueError, TypeError)):
            attention_packed(*args, out=bad)
    for bad in (torch.empty((Tq, Hq), dtype=torch.float32, device=dev),
                torch.empty((Hq, Tq), dtype=torch.float16, device=dev)):
        with pytest.raises((ValueError, TypeError)):
            attention_packed(*args, return_lse=True, lse=bad)
