"""GPU parity of the paged K/V entry point: the keys and values of a packed
input are scattered into shuffled pages (unused slots hold NaN), the HIP path
runs on the pages, and its result is compared with the float64 oracle on the
packed input."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from mea_workloads import generate, random_case, to_fp8, to_paged
from parity import compare, compare_rows, oracle_full

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def run_paged(inp, page_size, seed=0):
    from memory_efficient_attention_amd import attention_paged
    pk = to_paged(inp, page_size, seed=seed)
    dev = "cuda"
    q = inp.q.to(dev)
    out = torch.full_like(q, float("nan"))
    res = attention_paged(q, pk.k_cache.to(dev), pk.v_cache.to(dev), pk.block_table.to(dev),
                          inp.seqstart_q.to(dev), inp.seqstart_k.to(dev), inp.max_seqlen_q,
                          inp.max_seqlen_k, causal=inp.causal,
                          alibi_slopes=None if inp.alibi_slopes is None else inp.alibi_slopes.to(dev),
                          scale=inp.scale, return_lse=True, out=out, total_k=inp.total_k)
    torch.cuda.synchronize()
    return res[0].cpu(), res[1].cpu()


PAGED_CASES = [
    # (seqlens_q, seqlens_k, Hq, Hkv, D, dtype, causal, alibi, page_size)
    ([1] * 6, [1, 63, 64, 65, 300, 1000], 16, 4, 128, "bf16", False, True, 64),      # decode
    ([1] * 5, [700, 0, 129, 2000, 64], 8, 8, 64, "fp16", True, False, 128),          # decode, empty
    ([1] * 3, [5000, 4100, 33], 40, 1, 128, "bf16", False, False, 256),              # decode, MQA
    ([37, 120, 8, 200], None, 8, 8, 64, "fp16", True, False, 64),                    # prefill
    ([200, 17, 300], None, 12, 4, 128, "bf16", True, True, 128),                     # prefill, GQA 3
    ([40, 7, 90], [100, 7, 300], 8, 2, 128, "bf16", True, True, 64),                 # L_q < L_k
    ([2, 1, 5], [500, 400, 65], 8, 2, 128, "bf16", True, False, 192),                # mixed lengths
]


@pytest.mark.parametrize("ci", range(len(PAGED_CASES)))
def test_paged_cases(ci):
    lq, lk, Hq, Hkv, D, dt, causal, alibi, ps = PAGED_CASES[ci]
    inp = random_case(3000 + ci, lq, lk, Hq=Hq, Hkv=Hkv, D=D, dtype=dt, causal=causal, alibi=alibi)
    _log(f"paged {ci}: {PAGED_CASES[ci]}")
    out, lse = run_paged(inp, ps, seed=ci)
    ref_out, ref_lse = oracle_full(inp)
    _log(f"  {compare(out, lse, ref_out, ref_lse, dt, f'paged {ci}')}")


def test_paged_decode_full_size_sampled():
    inp = generate("decode_splitkv_64req_h64kv8_d128_bf16")
    _log(f"paged decode 64 requests, sum Lk={inp.total_k}, page 64")
    out, lse = run_paged(inp, 64)
    rows = [(t, h) for t in range(64) for h in (0, 9, 63)]
    _log(f"  {compare_rows(out, lse, inp, rows, 'paged decode sampled')}")


def test_paged_prefill_first_sequences_full():
    inp = generate("varlen_causal_gqa_64seq_h32kv8_d128_bf16", num_seqs=5, alibi=True)
    _log(f"paged prefill first 5 sequences, lengths {inp.seqlens_q}, page 128")
    out, lse = run_paged(inp, 128)
    ref_out, ref_lse = oracle_full(inp)
    _log(f"  {compare(out, lse, ref_out, ref_lse, 'bf16', 'paged prefill 5 seqs')}")


# ---------------------------------------------------------------- fp8 caches
def run_paged_fp8(inp, page_size, seed=0, out_dtype=torch.bfloat16):
    """q, k, v quantised to e4m3 (per-tensor scales); the k/v codes scattered
    into shuffled pages (unused slots hold the e4m3 NaN code); returns the
    GPU result and the fp8 inputs the oracle is to see."""
    from memory_efficient_attention_amd import attention_paged_fp8
    f = to_fp8(inp)
    pk = to_paged(dataclasses.replace(inp, k=f.k8, v=f.v8), page_size, seed=seed)
    dev = "cuda"
    out = torch.full((inp.total_q, inp.Hq, inp.D), float("nan"), dtype=out_dtype, device=dev)
    res = attention_paged_fp8(f.q8.to(dev), pk.k_cache.to(dev), pk.v_cache.to(dev), f.q_scale, f.k_scale, f.v_scale,
                              pk.block_table.to(dev), inp.seqstart_q.to(dev), inp.seqstart_k.to(dev),
                              inp.max_seqlen_q, inp.max_seqlen_k, causal=inp.causal,
                              alibi_slopes=None if inp.alibi_slopes is None else inp.alibi_slopes.to(dev),
                              scale=inp.scale, out_dtype=out_dtype, return_lse=True, out=out, total_k=inp.total_k)
    torch.cuda.synchronize()
    return res[0].cpu(), res[1].cpu(), f


def oracle_fp8(inp, f):
    return oracle.attention_forward_fp8(f.q8, f.k8, f.v8, f.q_scale, f.k_scale, f.v_scale, inp.seqstart_q,
                                        inp.seqstart_k, causal=inp.causal, alibi_slopes=inp.alibi_slopes,
                                        scale=inp.scale)


PAGED_FP8_CASES = [
    # (seqlens_q, seqlens_k, Hq, Hkv, causal, alibi, page_size, out dtype)
    ([1] * 6, [1, 63, 64, 65, 300, 1000], 16, 4, False, True, 64, torch.bfloat16),     # decode
    ([1] * 5, [700, 0, 129, 2000, 64], 8, 8, True, False, 128, torch.float16),         # decode, empty
    ([1] * 3, [5000, 4100, 33], 40, 1, False, False, 256, torch.bfloat16),             # decode, MQA
    ([1] * 4, [95, 130, 2000, 191], 64, 8, True, False, 64, torch.bfloat16),           # decode, group 8
    ([200, 17, 300], None, 12, 4, True, True, 128, torch.bfloat16),                    # prefill, GQA 3
    ([40, 7, 90], [100, 7, 300], 8, 2, True, True, 64, torch.float16),                 # L_q < L_k
]


@pytest.mark.parametrize("ci", range(len(PAGED_FP8_CASES)))
def test_paged_fp8_cases(ci):
    lq, lk, Hq, Hkv, causal, alibi, ps, odt = PAGED_FP8_CASES[ci]
    inp = random_case(3100 + ci, lq, lk, Hq=Hq, Hkv=Hkv, D=128, dtype="bf16", causal=causal, alibi=alibi)
    _log(f"paged fp8 {ci}: {PAGED_FP8_CASES[ci][:-1]}")
    out, lse, f = run_paged_fp8(inp, ps, seed=ci, out_dtype=odt)
    ref_out, ref_lse = oracle_fp8(inp, f)
    _log(f"  {compare(out, lse, ref_out, ref_lse, 'bf16' if odt == torch.bfloat16 else 'fp16', f'paged fp8 {ci}')}")


def test_paged_fp8_decode_full_size_sampled():
    """The 64-request decode workload in e4m3 on shuffled 64-key pages; sampled rows."""
    inp = generate("decode_splitkv_64req_h64kv8_d128_bf16")
    _log(f"paged fp8 decode 64 requests, sum Lk={inp.total_k}, page 64")
    out, lse, f = run_paged_fp8(inp, 64)
    assert not torch.isnan(out).any()
    rows = [(t, h) for t in range(64) for h in (0, 9, 63)]
    q = f.q8.to(torch.float64) * f.q_scale
    k = f.k8.to(torch.float64) * f.k_scale
    v = f.v8.to(torch.float64) * f.v_scale
    ro, rl = oracle.attention_rows(q, k, v, inp.seqstart_q, inp.seqstart_k, rows, causal=inp.causal, scale=inp.scale)
    go = torch.stack([out[t, h] for t, h in rows])
    gl = torch.stack([lse[h, t] for t, h in rows])
    _log(f"  {compare(go, gl, ro, rl, 'bf16', 'paged fp8 decode sampled')}")


# ------------------------------------------------------ out-of-range entries
BAD_PAGE_CASES = [
    # (seqlens_q, seqlens_k, Hq, Hkv, D, dtype, causal, alibi, page_size, fp8, {(sequence, block): entry})
    ([1] * 4, [300, 64, 1000, 129], 16, 4, 128, "bf16", True, True, 64, False,
     {(0, 2): "num_pages", (2, 0): -1, (2, 15): 2**31 - 1, (3, 2): "num_pages+5"}),              # decode
    ([37, 120, 200], None, 8, 2, 64, "fp16", True, False, 64, False,
     {(1, 1): -1, (2, 0): "num_pages", (2, 3): 2**31 - 1}),                                     # prefill
    ([1] * 4, [300, 64, 1000, 129], 16, 4, 128, "bf16", True, False, 64, True,
     {(0, 2): "num_pages", (2, 0): -1, (2, 15): 2**31 - 1}),                                    # fp8 decode
    ([40, 7, 90], [100, 7, 300], 8, 2, 128, "bf16", True, True, 64, True,
     {(0, 1): "num_pages", (2, 2): -1}),                                                       # fp8 prefill
]


def _zero_blocks(x, inp, blocks, page_size):
    x = x.clone()
    sk = inp.seqstart_k.tolist()
    for b, i in blocks:
        x[sk[b] + i * page_size:min(sk[b] + (i + 1) * page_size, sk[b + 1])] = 0
    return x


@pytest.mark.parametrize("ci", range(len(BAD_PAGE_CASES)))
def test_out_of_range_entries_read_as_zeros(ci):
    """Block-table entries outside [0, num_pages) (num_pages itself, past it,
    -1 and 2^31 - 1) are never dereferenced: the keys and values of those
    blocks read as zeros.  The result equals the oracle on the packed input
    with those keys and values set to zero (e4m3 code 0 is +0)."""
    from memory_efficient_attention_amd import attention_paged, attention_paged_fp8
    lq, lk, Hq, Hkv, D, dt, causal, alibi, ps, fp8, bad = BAD_PAGE_CASES[ci]
    inp = random_case(3200 + ci, lq, lk, Hq=Hq, Hkv=Hkv, D=D, dtype=dt, causal=causal, alibi=alibi)
    _log(f"out-of-range block-table entries {ci}: {bad}")
    dev = "cuda"
    slopes = None if inp.alibi_slopes is None else inp.alibi_slopes.to(dev)
    if fp8:
        f = to_fp8(inp)
        pk = to_paged(dataclasses.replace(inp, k=f.k8, v=f.v8), ps, seed=ci)
    else:
        pk = to_paged(inp, ps, seed=ci)
    num_pages = pk.k_cache.shape[0]
    table = pk.block_table.clone()
    for (b, i), e in bad.items():
        assert i * ps < inp.seqlens_k[b]
        table[b, i] = {"num_pages": num_pages, "num_pages+5": num_pages + 5}.get(e, e)
    out = torch.full((inp.total_q, Hq, D), float("nan"), dtype=torch.bfloat16 if dt == "bf16" else torch.float16,
                     device=dev)
    common = dict(causal=causal, alibi_slopes=slopes, scale=inp.scale, return_lse=True, out=out, total_k=inp.total_k)
    if fp8:
        res = attention_paged_fp8(f.q8.to(dev), pk.k_cache.to(dev), pk.v_cache.to(dev), f.q_scale, f.k_scale,
                                  f.v_scale, table.to(dev), inp.seqstart_q.to(dev), inp.seqstart_k.to(dev),
                                  inp.max_seqlen_q, inp.max_seqlen_k, out_dtype=out.dtype, **common)
    else:
        res = attention_paged(inp.q.to(dev), pk.k_cache.to(dev), pk.v_cache.to(dev), table.to(dev),
                              inp.seqstart_q.to(dev), inp.seqstart_k.to(dev), inp.max_seqlen_q, inp.max_seqlen_k,
                              **common)
    torch.cuda.synchronize()
    got_out, got_lse = res[0].cpu(), res[1].cpu()
    if fp8:
        fz = dataclasses.replace(f, k8=_zero_blocks(f.k8, inp, bad, ps), v8=_zero_blocks(f.v8, inp, bad, ps))
        ref_out, ref_lse = oracle_fp8(inp, fz)
    else:
        inz = dataclasses.replace(inp, k=_zero_blocks(inp.k, inp, bad, ps), v=_zero_blocks(inp.v, inp, bad, ps))
        ref_out, ref_lse = oracle_full(inz)
    _log(f"  {compare(got_out, got_lse, ref_out, ref_lse, dt, f'out-of-range entries {ci}')}")


# ---------------------------------------------------------------- persistent prefill grid on pages
def _many_short_sequences(seed, dtype, alibi):
    """240 sequences, one of 2,048 queries, the rest U[0, 150) with every 17th
    empty: 240 x 32 query-tile slots per key/value head, enough for the
    persistent prefill grid.  std 0.5 keeps |out| below 4 (a few keys make a
    row's output close to one V row), where half a bfloat16 ulp is within the
    1e-2 bound."""
    rng = np.random.default_rng(91)
    lq = [int(x) for x in rng.integers(0, 150, size=240)]
    lq = [0 if i % 17 == 3 else L for i, L in enumerate(lq)]
    lq[100] = 2048
    lk = [L + int(e) for L, e in zip(lq, rng.integers(0, 40, size=240))]
    return random_case(seed, lq, lk, Hq=32, Hkv=8, D=128, dtype=dtype, causal=True, alibi=alibi, std=0.5)


def test_paged_persistent_prefill():
    inp = _many_short_sequences(4620, "bf16", True)
    _log(f"paged persistent prefill: T={inp.total_q}, page 128")
    out, lse = run_paged(inp, 128, seed=5)
    ref_out, ref_lse = oracle_full(inp)
    _log(f"  {compare(out, lse, ref_out, ref_lse, 'bf16', 'paged persistent prefill')}")


def test_paged_fp8_persistent_prefill():
    inp = _many_short_sequences(4630, "bf16", False)
    _log(f"paged fp8 persistent prefill: T={inp.total_q}, page 64")
    out, lse, f = run_paged_fp8(inp, 64, seed=6)
    ref_out, ref_lse = oracle_fp8(inp, f)
    _log(f"  {compare(out, lse, ref_out, ref_lse, 'bf16', 'paged fp8 persistent prefill')}")
