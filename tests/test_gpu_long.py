"""GPU parity at the size limits of the C ABI, on sampled rows (the oracle
computes each sampled row on its own):
- one causal prefill sequence of 131,072 tokens (GQA 8/2, D 128, ALiBi);
- decode over one sequence of 1,048,575 keys x 8 key/value heads x D 128,
  the longest that keeps a sequence's key rows below 2^31 bytes (the
  library addresses them with 32-bit offsets), in bf16 and in fp8;
- 65,535 short sequences, the largest num_seqs the library accepts."""
import sys

import pytest
import torch

import oracle
from mea_workloads import random_case, sample_rows, to_fp8
from parity import compare, compare_rows, run_gpu

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def test_prefill_one_sequence_131072_tokens():
    inp = random_case(6100, [131072], Hq=8, Hkv=2, D=128, dtype="bf16", causal=True, alibi=True)
    _log("long prefill: 1 x 131072 tokens, Hq 8 / Hkv 2, D 128, causal + ALiBi")
    out, lse = run_gpu(inp)
    rows = [(0, 0), (1, 3), (4095, 7), (65536, 2), (131070, 5), (131071, 0), (131071, 7)] + sample_rows(inp, 25, seed=4)
    _log(f"  {compare_rows(out, lse, inp, rows, 'prefill 131072')}")


MAX_KEYS = (1 << 31) // (8 * 128 * 2) - 1   # 1,048,575 keys of 8 heads x 128 bf16 values


@pytest.fixture(scope="module")
def long_decode():
    inp = random_case(6200, [1], [MAX_KEYS], Hq=64, Hkv=8, D=128, dtype="bf16")
    rows = [(0, h) for h in (0, 7, 8, 31, 40, 63)]
    return inp, rows


def test_decode_at_the_offset_limit_bf16(long_decode):
    inp, rows = long_decode
    _log(f"long decode: 1 query over {MAX_KEYS} keys, Hq 64 / Hkv 8, D 128, bf16")
    out, lse = run_gpu(inp)
    _log(f"  {compare_rows(out, lse, inp, rows, 'decode at the offset limit')}")


def test_decode_at_the_offset_limit_fp8(long_decode):
    from memory_efficient_attention_amd import attention_packed_fp8
    inp, rows = long_decode
    f = to_fp8(inp)
    _log(f"long decode fp8: 1 query over {MAX_KEYS} keys, Hq 64 / Hkv 8, D 128")
    dev = "cuda"
    out, lse = attention_packed_fp8(f.q8.to(dev), f.k8.to(dev), f.v8.to(dev), f.q_scale, f.k_scale, f.v_scale,
                                    inp.seqstart_q.to(dev), inp.seqstart_k.to(dev), inp.max_seqlen_q,
                                    inp.max_seqlen_k, scale=inp.scale, return_lse=True)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    # the oracle on the dequantised values of key/value heads 0 and 7 only
    # (query heads 0..7 and 56..63), so that it holds 2 of the 8 heads in float64
    qh = list(range(8)) + list(range(56, 64))
    q = f.q8[:, qh].to(torch.float64) * f.q_scale
    k = f.k8[:, [0, 7]].to(torch.float64) * f.k_scale
    v = f.v8[:, [0, 7]].to(torch.float64) * f.v_scale
    picks = [(0, 0), (0, 5), (0, 56), (0, 63)]
    ro, rl = oracle.attention_rows(q, k, v, inp.seqstart_q, inp.seqstart_k, [(t, qh.index(h)) for t, h in picks],
                                   causal=False, scale=inp.scale)
    go = torch.stack([out[t, h] for t, h in picks])
    gl = torch.stack([lse[h, t] for t, h in picks])
    _log(f"  {compare(go, gl, ro, rl, 'bf16', 'fp8 decode at the offset limit')}")


def test_65535_sequences():
    import numpy as np
    rng = np.random.default_rng(6300)
    lens = rng.integers(0, 7, size=65535).tolist()
    inp = random_case(6300, lens, Hq=4, Hkv=2, D=64, dtype="fp16", causal=True)
    _log(f"65535 sequences, {inp.total_q} tokens")
    out, lse = run_gpu(inp)
    assert not torch.isnan(out).any()
    _log(f"  {compare_rows(out, lse, inp, sample_rows(inp, 96, seed=6), '65535 sequences')}")
