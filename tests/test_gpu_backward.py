"""GPU parity of the backward (dq, dk, dv): the HIP kernels against the CPU
float64 oracle's chain-rule gradients on the same seeded inputs and upstream
gradient, element by element; at the full benchmark size, whole sequences
sampled from the packed batch (sequences are independent)."""
import dataclasses
import sys

import pytest
import torch

from mea_workloads import Inputs, generate, random_case, random_dout, seqstart_from_lengths
from parity import compare_grads, oracle_backward, run_gpu_backward, to_device

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


CASES = [
    # (name, seqlens_q, seqlens_k, Hq, Hkv, D, dtype, causal, alibi)
    ("varlen_fp16_d64", [37, 120, 8, 200], None, 8, 8, 64, "fp16", False, False),
    ("varlen_fp16_d64_causal", [37, 120, 8, 200], None, 8, 8, 64, "fp16", True, False),
    ("gqa_bf16_d128_causal_alibi", [130, 1, 77, 300], None, 8, 2, 128, "bf16", True, True),
    ("gqa_bf16_d128_alibi", [130, 1, 77, 300], None, 8, 2, 128, "bf16", False, True),
    ("mqa_fp16_d128", [256, 129], None, 8, 1, 128, "fp16", False, False),
    ("mqa_bf16_d64_causal_alibi", [256, 129, 64], None, 6, 1, 64, "bf16", True, True),
    ("lq_gt_lk_causal", [3, 5, 70, 150], [7, 2, 200, 64], 4, 2, 64, "bf16", True, False),
    ("lq_lt_lk_causal_alibi", [65, 17, 200], [300, 17, 333], 4, 4, 128, "fp16", True, True),
    ("empty_sides", [0, 65, 10, 0, 33], [5, 0, 10, 0, 129], 4, 2, 128, "bf16", True, False),
    ("decode_shaped", [1, 1, 1, 1], [300, 1, 64, 1000], 8, 2, 128, "bf16", True, True),
    ("long_2x1024_causal", [1024, 1024], None, 8, 2, 128, "bf16", True, False),
]


def _case(ci, seed):
    name, lq, lk, Hq, Hkv, D, dtype, causal, alibi = CASES[ci]
    inp = random_case(seed, lq, lk, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, causal=causal, alibi=alibi)
    return inp, random_dout(seed, inp)


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_backward_parity(ci):
    inp, dout = _case(ci, seed=500 + ci)
    _log(f"backward {CASES[ci][0]}")
    got = run_gpu_backward(inp, dout)
    ref = oracle_backward(inp, dout)
    _log(f"  {compare_grads(got, ref, inp.dtype, CASES[ci][0])}")


def test_backward_is_deterministic():
    """No atomics: two calls give bitwise equal gradients."""
    inp, dout = _case(2, seed=600)
    dev = to_device(inp)
    a = run_gpu_backward(inp, dout, dev)
    b = run_gpu_backward(inp, dout, dev)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_autograd_through_memory_efficient_attention():
    """loss.backward() through the xFormers-style call reaches the HIP backward."""
    from memory_efficient_attention_amd import BlockDiagonalCausalMask, memory_efficient_attention
    inp = random_case(7, [100, 37, 64], Hq=8, Hkv=2, D=64, dtype="bf16", causal=True)
    dout = random_dout(7, inp)
    _log("autograd")
    q = inp.q.cuda().unsqueeze(0).requires_grad_()
    k = inp.k.cuda().unsqueeze(0).requires_grad_()
    v = inp.v.cuda().unsqueeze(0).requires_grad_()
    mask = BlockDiagonalCausalMask.from_seqlens(inp.seqlens_q)
    out = memory_efficient_attention(q, k, v, attn_bias=mask, scale=inp.scale)
    out.backward(dout.cuda().unsqueeze(0))
    torch.cuda.synchronize()
    got = (q.grad[0].cpu(), k.grad[0].cpu(), v.grad[0].cpu())
    _log(f"  {compare_grads(got, oracle_backward(inp, dout), 'bf16', 'autograd')}")


def _one_sequence(inp: Inputs, b: int, dout: torch.Tensor):
    sq, sk = inp.seqstart_q.tolist(), inp.seqstart_k.tolist()
    lq, lk = sq[b + 1] - sq[b], sk[b + 1] - sk[b]
    sub = dataclasses.replace(inp, q=inp.q[sq[b]:sq[b + 1]], k=inp.k[sk[b]:sk[b + 1]], v=inp.v[sk[b]:sk[b + 1]],
                              seqstart_q=seqstart_from_lengths([lq]), seqstart_k=seqstart_from_lengths([lk]),
                              seqlens_q=[lq], seqlens_k=[lk], bmghk=None)
    return sub, dout[sq[b]:sq[b + 1]]


@pytest.mark.parametrize("alibi", [False, True])
def test_backward_full_size_sampled_sequences(alibi):
    """All 64 sequences (137,663 tokens, 32 q / 8 kv heads, D=128, bf16,
    causal) on the GPU in one call; the oracle checks whole sequences (every
    dq, dk, dv row of them): the shortest, one near 1,000 tokens and one
    near 2,000."""
    inp = generate("varlen_causal_gqa_64seq_h32kv8_d128_bf16", alibi=alibi)
    dout = random_dout(3, inp)
    _log(f"backward full size alibi={alibi} T={inp.total_q}")
    dq, dk, dv = run_gpu_backward(inp, dout)
    for g in (dq, dk, dv):
        assert not torch.isnan(g).any()
    lens = inp.seqlens_q
    picks = {min(range(len(lens)), key=lambda i: lens[i]),
             min(range(len(lens)), key=lambda i: abs(lens[i] - 1000)),
             min(range(len(lens)), key=lambda i: abs(lens[i] - 2000))}
    sq, sk = inp.seqstart_q.tolist(), inp.seqstart_k.tolist()
    for b in sorted(picks):
        sub, sub_dout = _one_sequence(inp, b, dout)
        ref = oracle_backward(sub, sub_dout)
        got = (dq[sq[b]:sq[b + 1]], dk[sk[b]:sk[b + 1]], dv[sk[b]:sk[b + 1]])
        _log(f"  seq {b} (L={lens[b]}): {compare_grads(got, ref, 'bf16', f'full size seq {b}')}")
