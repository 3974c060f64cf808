"""GPU parity of mixed batches (prefills followed by one-query decode steps,
a serving engine's layout) through mea_fwd_mixed, which serves the prefills
with the prefill kernels and the decode steps with the split-KV kernels in
one call; checked element by element against the float64 oracle on the whole
batch, at full size on sampled rows, and routed automatically by
``memory_efficient_attention`` from the mask's host lengths."""
import sys

import pytest
import torch

from memory_efficient_attention_amd import BlockDiagonalCausalMask, BlockDiagonalMask
from mea_workloads import mixed_case, random_case, sample_rows
from parity import compare, compare_rows, oracle_full, to_device

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _mask(inp):
    cls = BlockDiagonalCausalMask if inp.causal else BlockDiagonalMask
    return cls.from_seqlens(inp.seqlens_q, inp.seqlens_k)


def run_mixed(inp, dev=None):
    from memory_efficient_attention_amd import attention_packed
    d = dev or to_device(inp)
    mixed = _mask(inp).mixed_split()
    assert mixed is not None
    out = torch.full_like(d["q"], float("nan"))
    out, lse = attention_packed(d["q"], d["k"], d["v"], d["seqstart_q"], d["seqstart_k"], inp.max_seqlen_q,
                                inp.max_seqlen_k, causal=inp.causal, alibi_slopes=d["slopes"], scale=inp.scale,
                                return_lse=True, out=out, mixed=mixed)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


CASES = [
    # (seqlens_q, seqlens_k, Hq, Hkv, D, dtype, causal, alibi)
    ([130, 7, 64, 1, 1, 1, 1, 1], [130, 7, 64, 900, 33, 1000, 1, 4000], 8, 2, 128, "bf16", True, True),
    ([37, 120, 8, 1, 1], [37, 120, 8, 200, 65], 8, 8, 64, "fp16", False, False),
    ([40, 17, 1, 1, 1], [100, 17, 0, 64, 3000], 8, 2, 128, "bf16", True, False),    # L_q < L_k, empty keys
    ([256, 1, 1], [256, 5000, 4100], 16, 1, 128, "bf16", False, True),               # MQA
    ([1, 300, 1, 1], [500, 300, 129, 700], 12, 4, 64, "bf16", True, True),            # a 1-query prefill first
    ([0, 65, 1, 1], [5, 65, 2048, 31], 8, 4, 128, "fp16", True, False),               # empty prefill
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_mixed_parity(ci):
    lq, lk, Hq, Hkv, D, dt, causal, alibi = CASES[ci]
    inp = random_case(5000 + ci, lq, lk, Hq=Hq, Hkv=Hkv, D=D, dtype=dt, causal=causal, alibi=alibi)
    _log(f"mixed {ci}: {CASES[ci]}")
    out, lse = run_mixed(inp)
    ref_out, ref_lse = oracle_full(inp)
    _log(f"  {compare(out, lse, ref_out, ref_lse, dt, f'mixed {ci}')}")


def test_mixed_routed_by_memory_efficient_attention():
    """The xFormers-style call on a [1, T, H, D] mixed batch takes the mixed
    path (bitwise the result of attention_packed(mixed=...))."""
    from memory_efficient_attention_amd import memory_efficient_attention
    inp = random_case(5100, [100, 37, 1, 1, 1], [100, 37, 800, 70, 3000], Hq=8, Hkv=2, D=64, dtype="bf16",
                      causal=True)
    d = to_device(inp)
    out = memory_efficient_attention(d["q"][None], d["k"][None], d["v"][None], attn_bias=_mask(inp),
                                     scale=inp.scale)
    torch.cuda.synchronize()
    ref, _ = run_mixed(inp, d)
    assert torch.equal(out[0].cpu(), ref)


def test_mixed_full_size_sampled():
    """8 prefills U[128, 4096] + 56 decode steps over U[1024, 32768] keys, 32/8
    heads, D 128, bf16, causal (the mixed serving workload): sampled rows of
    both parts against the oracle."""
    inp = mixed_case(0)
    _log(f"mixed full size: Tq={inp.total_q} Tk={inp.total_k}")
    out, lse = run_mixed(inp)
    rows = sample_rows(inp, 48, seed=3)
    n_pre = _mask(inp).mixed_split()[1]
    rows += [(t, h) for t in range(n_pre, inp.total_q, 7) for h in (0, inp.Hq - 1)]   # decode rows
    _log(f"  {compare_rows(out, lse, inp, sorted(set(rows)), 'mixed full size')}")


def test_mixed_with_a_persistent_prefill_part():
    """240 prefills (one of 2,048 queries, the rest U[2, 150), enough query-tile
    slots for the persistent prefill grid) followed by 24 decode steps over
    U[1, 3000] keys: the persistent workgroups on the first sequences, then the
    split-KV kernels from the decode part's sequence and key bases.  std 0.5
    keeps |out| below 4 (half a bfloat16 ulp within the 1e-2 bound)."""
    import numpy as np
    rng = np.random.default_rng(97)
    lq = [int(x) for x in rng.integers(2, 150, size=240)]
    lq[100] = 2048
    lk = [L + int(e) for L, e in zip(lq, rng.integers(0, 40, size=240))]
    lq += [1] * 24
    lk += [int(x) for x in rng.integers(1, 3000, size=24)]
    inp = random_case(5200, lq, lk, Hq=32, Hkv=8, D=128, dtype="bf16", causal=True, alibi=True, std=0.5)
    split = _mask(inp).mixed_split()
    assert split[0] == 240
    _log(f"mixed, persistent prefill part: Tq={inp.total_q} Tk={inp.total_k} split={split}")
    out, lse = run_mixed(inp)
    ref_out, ref_lse = oracle_full(inp)
    _log(f"  {compare(out, lse, ref_out, ref_lse, 'bf16', 'mixed persistent')}")
