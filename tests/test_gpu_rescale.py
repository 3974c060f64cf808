"""GPU parity when the online softmax has to rescale its running sums many
times: key rows grow in magnitude toward the start of each sequence, so the
running row maximum keeps rising as the kernels walk key tiles from the
causal diagonal back to the start, by more than the 2^8 that triggers a
rescale, at different tiles for different query rows.  This exercises the
rescale of the row sums kept on the matrix cores (ALiBi, fp8: lane n < 16
holds the sums of queries n and n + 16, each with its own factor) and of the
per-lane sums (bf16/fp16 without ALiBi), against the float64 oracle."""
import math
import sys

import pytest
import torch

import oracle
from mea_workloads import random_case, to_fp8
from parity import compare, oracle_full, run_gpu

pytestmark = pytest.mark.gpu

RAMP = 5.0   # the first key of a sequence is 1 + RAMP times larger than the last


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _ramped(inp):
    """``inp`` with key row j of a sequence of L keys scaled by 1 + RAMP (1 - j / L),
    and V halved (exactly): the weights concentrate on a few keys, so a row's
    output is close to one V row, and with |V| mostly below 4 half a bfloat16
    ulp of it (at most 2^-7) stays within the 1e-2 bound."""
    k = inp.k.double().clone()
    sk = inp.seqstart_k.tolist()
    for b in range(len(sk) - 1):
        L = sk[b + 1] - sk[b]
        if L:
            f = 1.0 + RAMP * (1.0 - torch.arange(L, dtype=torch.float64) / L)
            k[sk[b]:sk[b + 1]] *= f[:, None, None]
    inp.k = k.to(inp.k.dtype)
    inp.v = inp.v * 0.5
    return inp


def _rescales(inp, b, h):
    """How many 64-key tiles, walked from the causal diagonal backwards, raise
    the running maximum of some query row of sequence b, head h by more than
    8 in log2 units (float64 scores; the ALiBi bias included): the case must
    need several."""
    sq, sk = inp.seqstart_q.tolist(), inp.seqstart_k.tolist()
    Lq, Lk = sq[b + 1] - sq[b], sk[b + 1] - sk[b]
    g = h // (inp.Hq // inp.Hkv)
    s = inp.q[sq[b]:sq[b + 1], h].double() @ inp.k[sk[b]:sk[b + 1], g].double().T * inp.scale
    qpos = torch.arange(Lq)[:, None] + (Lk - Lq)
    kpos = torch.arange(Lk)[None, :]
    if inp.alibi_slopes is not None:
        s = s - float(inp.alibi_slopes[h]) * (qpos - kpos).abs()
    if inp.causal:
        s = s.masked_fill(kpos > qpos, -math.inf)
    s = s * math.log2(math.e)
    count = 0
    m = torch.full((Lq,), -math.inf, dtype=torch.float64)
    for t in range((Lk + 63) // 64 - 1, -1, -1):
        mt = s[:, 64 * t:64 * t + 64].max(dim=1).values
        if bool(((mt > m + 8) & torch.isfinite(m)).any()):
            count += 1
        m = torch.maximum(m, mt)
    return count


CASES = [
    # (name, seqlens, Hq, Hkv, D, dtype, causal, alibi, fp8)
    ("bf16_causal_alibi_gqa", [300, 700, 65], 8, 2, 128, "bf16", True, True, False),
    ("bf16_alibi_noncausal", [257, 400], 8, 2, 128, "bf16", False, True, False),
    ("fp16_causal_d64", [500, 129], 4, 4, 64, "fp16", True, False, False),
    ("bf16_causal_d128", [640, 33], 8, 8, 128, "bf16", True, False, False),
    ("fp8_causal_alibi_gqa", [300, 700], 8, 2, 128, "bf16", True, True, True),
    ("fp8_causal", [640, 97], 8, 4, 128, "bf16", True, False, True),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_many_rescales(ci):
    name, lens, Hq, Hkv, D, dtype, causal, alibi, fp8 = CASES[ci]
    inp = _ramped(random_case(8800 + ci, lens, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, causal=causal, alibi=alibi))
    longest = max(range(len(lens)), key=lambda i: lens[i])
    n = _rescales(inp, longest, Hq - 1)   # the head with the smallest ALiBi slope
    _log(f"rescale {name}: {n} tiles raise the maximum by more than 2^8 (sequence {longest}, head {Hq - 1})")
    assert n >= 2, f"{name}: the case needs several rescales, got {n}"
    if not fp8:
        out, lse = run_gpu(inp)
        ref_out, ref_lse = oracle_full(inp)
        _log(f"  {compare(out, lse, ref_out, ref_lse, dtype, name)}")
        return
    from memory_efficient_attention_amd import attention_packed_fp8
    f = to_fp8(inp)
    dev = "cuda"
    out = torch.full((inp.total_q, Hq, D), float("nan"), dtype=torch.bfloat16, device=dev)
    o, lse = attention_packed_fp8(f.q8.to(dev), f.k8.to(dev), f.v8.to(dev), f.q_scale, f.k_scale, f.v_scale,
                                  inp.seqstart_q.to(dev), inp.seqstart_k.to(dev), inp.max_seqlen_q, inp.max_seqlen_k,
                                  causal=causal, alibi_slopes=None if inp.alibi_slopes is None else
                                  inp.alibi_slopes.to(dev), scale=inp.scale, out_dtype=torch.bfloat16,
                                  return_lse=True, out=out)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.attention_forward_fp8(f.q8, f.k8, f.v8, f.q_scale, f.k_scale, f.v_scale,
                                                    inp.seqstart_q, inp.seqstart_k, causal=causal,
                                                    alibi_slopes=inp.alibi_slopes, scale=inp.scale)
    _log(f"  {compare(o.cpu(), lse.cpu(), ref_out, ref_lse, 'bf16', name)}")
