"""GPU parity for bfloat16 V outside the range where IEEE halves are exact.

The kernels feed P V with IEEE-half weights and bfloat16 V re-encoded as
halves, which is exact for 2^-14 <= |v| <= 65504.  A tile or block holding a
larger magnitude, or only smaller ones, keeps bfloat16 V and bfloat16
weights.  These cases plant such values into some sequences of a packed
batch (1e5, -1e30, all of a sequence's V scaled by 1e-6) next to untouched
control sequences, for prefill and decode, packed and paged, and compare with
the float64 oracle per (sequence, key/value head) at max-abs
<= 1e-2 * max|V| of that sequence and head (the relative form of the 1e-2
bfloat16 gate), lse within 1e-3 as usual.  Without the bfloat16 path the
planted values saturate at 65504 or lose their precision and fail this gate.
"""
import sys

import pytest
import torch

import oracle
from mea_workloads import random_case, to_paged

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _plant(inp, seed):
    """Sequence 0: one value 1e5; sequence 1: one value -1e30; sequence 2:
    its whole V scaled by 1e-6 (every value below 2^-14); the rest untouched."""
    g = torch.Generator().manual_seed(seed)
    v = inp.v.clone().float()
    sk = inp.seqstart_k.tolist()
    Hkv, D = v.shape[1], v.shape[2]
    for b, val in ((0, 1e5), (1, -1e30)):
        L = sk[b + 1] - sk[b]
        if L > 0:
            t = sk[b] + int(torch.randint(0, L, (1,), generator=g))
            v[t, int(torch.randint(0, Hkv, (1,), generator=g)), int(torch.randint(0, D, (1,), generator=g))] = val
    v[sk[2]:sk[3]] *= 1e-6
    inp.v = v.to(inp.v.dtype)
    return inp


def _check(out, lse, inp, what):
    ref_out, ref_lse = oracle.attention_forward(inp.q, inp.k, inp.v, inp.seqstart_q, inp.seqstart_k,
                                                causal=inp.causal, alibi_slopes=inp.alibi_slopes,
                                                scale=inp.scale)
    o = out.double()
    assert not torch.isnan(o).any(), f"{what}: NaN in out"
    sq, sk = inp.seqstart_q.tolist(), inp.seqstart_k.tolist()
    G = inp.Hq // inp.Hkv
    worst = 0.0
    for b in range(len(sq) - 1):
        if sq[b + 1] == sq[b]:
            continue
        for g in range(inp.Hkv):
            vmax = inp.v[sk[b]:sk[b + 1], g].double().abs().max().item() if sk[b + 1] > sk[b] else 0.0
            tol = 1e-2 * vmax if vmax > 0 else 1e-30
            err = (o[sq[b]:sq[b + 1], g * G:(g + 1) * G] - ref_out[sq[b]:sq[b + 1], g * G:(g + 1) * G]).abs().max().item()
            worst = max(worst, err / tol)
            assert err <= tol, f"{what}: sequence {b} head {g}: error {err:.3e} > 1e-2 * max|V| = {tol:.3e}"
    l = lse.double()
    fin = ~torch.isneginf(ref_lse)
    assert torch.equal(torch.isneginf(l), ~fin), f"{what}: -inf lse rows differ"
    lerr = (l[fin] - ref_lse[fin]).abs().max().item()
    assert lerr <= 1e-3, f"{what}: lse error {lerr:.3e}"
    return {"worst_err_over_tol": round(worst, 4), "max_abs_lse": lerr}


CASES = [
    # (seqlens_q, seqlens_k, Hq, Hkv, D, causal, alibi)
    ([130, 200, 64, 300], None, 8, 2, 128, True, False),        # prefill, GQA
    ([70, 129, 65, 33], None, 4, 4, 64, False, True),           # prefill, D 64, ALiBi
    ([1, 1, 1, 1], [1000, 3000, 64, 5000], 16, 2, 128, False, False),   # decode
    ([1, 1, 1, 1], [700, 65, 300, 2000], 8, 8, 64, False, True),        # decode, D 64, ALiBi
    ([40, 1, 90, 7], [100, 900, 300, 7], 8, 2, 128, True, True),        # mixed, L_q < L_k
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_bf16_v_out_of_half_range_packed(ci):
    from memory_efficient_attention_amd import attention_packed
    lq, lk, Hq, Hkv, D, causal, alibi = CASES[ci]
    inp = _plant(random_case(4100 + ci, lq, lk, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16", causal=causal,
                             alibi=alibi), seed=ci)
    _log(f"range packed {ci}: {CASES[ci]}")
    dev = "cuda"
    q = inp.q.to(dev)
    out = torch.full_like(q, float("nan"))
    out, lse = attention_packed(q, inp.k.to(dev), inp.v.to(dev), inp.seqstart_q.to(dev), inp.seqstart_k.to(dev),
                                inp.max_seqlen_q, inp.max_seqlen_k, causal=causal,
                                alibi_slopes=None if inp.alibi_slopes is None else inp.alibi_slopes.to(dev),
                                scale=inp.scale, return_lse=True, out=out)
    torch.cuda.synchronize()
    _log(f"  {_check(out.cpu(), lse.cpu(), inp, f'range packed {ci}')}")


def test_bf16_v_out_of_half_range_persistent():
    """The planted sequences in a batch large enough for the persistent
    prefill grid (240 sequences, one of 2,048 queries: 240 x 32 query-tile
    slots per key/value head): the second launch recomputes the items of the
    flagged tiles after the persistent workgroups have written them."""
    import numpy as np
    from memory_efficient_attention_amd import attention_packed
    rng = np.random.default_rng(93)
    lq = [300, 200, 130, 2048] + [int(x) for x in rng.integers(1, 150, size=236)]
    inp = _plant(random_case(4300, lq, None, Hq=32, Hkv=8, D=128, dtype="bf16", causal=True, alibi=True), seed=30)
    _log(f"range persistent: T={inp.total_q}")
    dev = "cuda"
    q = inp.q.to(dev)
    out, lse = attention_packed(q, inp.k.to(dev), inp.v.to(dev), inp.seqstart_q.to(dev), inp.seqstart_k.to(dev),
                                inp.max_seqlen_q, inp.max_seqlen_k, causal=True,
                                alibi_slopes=inp.alibi_slopes.to(dev), scale=inp.scale, return_lse=True,
                                out=torch.full_like(q, float("nan")))
    torch.cuda.synchronize()
    _log(f"  {_check(out.cpu(), lse.cpu(), inp, 'range persistent')}")


@pytest.mark.parametrize("ci", [0, 2, 4])
def test_bf16_v_out_of_half_range_paged(ci):
    from memory_efficient_attention_amd import attention_paged
    lq, lk, Hq, Hkv, D, causal, alibi = CASES[ci]
    inp = _plant(random_case(4200 + ci, lq, lk, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16", causal=causal,
                             alibi=alibi), seed=10 + ci)
    _log(f"range paged {ci}: {CASES[ci]}")
    pk = to_paged(inp, 128, seed=ci)
    dev = "cuda"
    q = inp.q.to(dev)
    out, lse = attention_paged(q, pk.k_cache.to(dev), pk.v_cache.to(dev), pk.block_table.to(dev),
                               inp.seqstart_q.to(dev), inp.seqstart_k.to(dev), inp.max_seqlen_q, inp.max_seqlen_k,
                               causal=causal,
                               alibi_slopes=None if inp.alibi_slopes is None else inp.alibi_slopes.to(dev),
                               scale=inp.scale, return_lse=True, out=torch.full_like(q, float("nan")),
                               total_k=inp.total_k)
    torch.cuda.synchronize()
    _log(f"  {_check(out.cpu(), lse.cpu(), inp, f'range paged {ci}')}")


def test_planted_inputs_need_the_bfloat16_path():
    """The planted values are outside the exact range of halves (so these
    tests would fail on a kernel that always re-encodes V as halves)."""
    inp = _plant(random_case(4100, [130, 200, 64, 300], None, Hq=8, Hkv=2, D=128, dtype="bf16"), seed=0)
    v = inp.v.float()
    sk = inp.seqstart_k.tolist()
    assert v[sk[0]:sk[1]].abs().max().item() > 65504 and v[sk[1]:sk[2]].abs().max().item() > 1e29
    assert 0 < v[sk[2]:sk[3]].abs().max().item() < 2.0 ** -14
