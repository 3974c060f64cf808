"""mea_fwd_noalloc (the forward without a caller workspace, for callers that
cannot allocate) against mea_fwd: the same call through both C entry points
gives bitwise the same out and lse, on calls in a row whose second is
smaller (the fixed scratch keeps the first call's contents), for prefill and
decode shapes; both also meet the oracle's gate."""
import sys

import pytest
import torch

from memory_efficient_attention_amd import _native, attention_packed
from mea_workloads import random_case
from parity import compare, oracle_full

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _noalloc(inp):
    dev = "cuda"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    ssq, ssk = inp.seqstart_q.to(dev), inp.seqstart_k.to(dev)
    slopes = None if inp.alibi_slopes is None else inp.alibi_slopes.to(dev)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((inp.Hq, inp.total_q), float("nan"), dtype=torch.float32, device=dev)
    code = _native.MEA_BF16 if inp.dtype == "bf16" else _native.MEA_F16
    stream = torch.cuda.current_stream()
    st = _native.mea_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                 ssq.data_ptr(), ssk.data_ptr(), len(inp.seqlens_q), inp.total_q, inp.total_k,
                                 inp.max_seqlen_q, inp.max_seqlen_k, inp.Hq, inp.Hkv, inp.D, code,
                                 int(inp.causal), None if slopes is None else slopes.data_ptr(), inp.scale,
                                 stream.cuda_stream)
    assert st == _native.MEA_OK, _native.mea_last_error()
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _with_workspace(inp):
    dev = "cuda"
    out, lse = attention_packed(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.seqstart_q.to(dev),
                                inp.seqstart_k.to(dev), inp.max_seqlen_q, inp.max_seqlen_k, causal=inp.causal,
                                alibi_slopes=None if inp.alibi_slopes is None else inp.alibi_slopes.to(dev),
                                scale=inp.scale, return_lse=True)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


PAIRS = [
    # two calls in a row, the second smaller: (seqlens_q, seqlens_k, Hq, Hkv, D, dtype, causal, alibi)
    (([2048, 2048, 1000], None, 16, 4, 128, "bf16", True, True),
     ([300, 17, 65], None, 16, 4, 128, "bf16", True, True)),
    (([1, 1, 1, 1], [20000, 3000, 65, 9000], 32, 8, 128, "bf16", False, False),
     ([1, 1], [700, 64], 32, 8, 128, "bf16", False, False)),
    (([37, 120, 8, 200], None, 8, 8, 64, "fp16", False, False),
     ([1, 1, 1], [1000, 7, 64], 8, 2, 64, "fp16", False, True)),
    # the first call has 8 x 20 x 64 = 10,240 work items, enough for the
    # persistent prefill grid (work counters in the fixed scratch), and needs
    # 11 MB of it
    (([4096] + [3] * 19, None, 32, 8, 128, "bf16", True, False),
     ([300, 17, 65], None, 32, 8, 128, "bf16", True, False)),
]


@pytest.mark.parametrize("pi", range(len(PAIRS)))
def test_noalloc_matches_workspace_entry_point(pi):
    for n, case in enumerate(PAIRS[pi]):
        lq, lk, Hq, Hkv, D, dt, causal, alibi = case
        inp = random_case(4700 + 10 * pi + n, lq, lk, Hq=Hq, Hkv=Hkv, D=D, dtype=dt, causal=causal, alibi=alibi)
        _log(f"noalloc pair {pi} call {n}: {case}")
        a_out, a_lse = _noalloc(inp)
        b_out, b_lse = _with_workspace(inp)
        assert torch.equal(a_out, b_out), "out differs from mea_fwd's"
        assert torch.equal(a_lse.isnan(), b_lse.isnan()) and torch.equal(a_lse[~a_lse.isnan()], b_lse[~b_lse.isnan()])
        ref_out, ref_lse = oracle_full(inp)
        _log(f"  {compare(a_out, a_lse, ref_out, ref_lse, dt, f'noalloc {pi}/{n}')}")


def test_noalloc_rejects_a_call_beyond_its_scratch():
    inp = random_case(4800, [1, 1], [3000, 5], Hq=8, Hkv=8, D=128, dtype="bf16")
    dev = "cuda"
    st = _native.mea_fwd_noalloc(1 << 20, 1 << 20, 1 << 20, 1 << 20, None, 1 << 20, 1 << 20, 64, 137663, 137663,
                                 4085, 4085, 32, 8, 128, _native.MEA_BF16, 1, None, 0.088,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == _native.MEA_ERR_UNSUPPORTED and "scratch" in _native.mea_last_error()
    _noalloc(inp)   # and the next call still works
