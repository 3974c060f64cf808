"""A seeded random sweep over the parameter space of the HIP paths, against
the CPU float64 oracle: every forward entry point (16-bit packed, 16-bit
paged, fp8 packed, fp8 paged) on drawn head counts and GQA ratios, head
dimensions, dtypes, masks, ALiBi, page sizes and length mixes (prefill,
decode and mixed; empty and 1-key sequences included), and the backward on
drawn 16-bit cases.  Each case is small enough for the oracle to finish in
about a second, and each prints its configuration before it runs."""
import dataclasses
import random
import sys

import pytest
import torch

import oracle
from mea_workloads import random_case, random_dout, to_fp8, to_paged
from parity import compare, compare_grads, oracle_backward, oracle_full, run_gpu, run_gpu_backward

pytestmark = pytest.mark.gpu

N_FORWARD = 120
N_BACKWARD = 24


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _lengths(rng, kind):
    n = rng.randint(1, 6)
    pick = lambda hi: rng.choice([0, 1, rng.randint(1, hi), rng.randint(1, hi)])
    if kind == "prefill":
        lq = [pick(300) for _ in range(n)]
        return lq, list(lq)
    if kind == "decode":
        return [rng.choice([0, 1, 1, 1]) for _ in range(n)], [pick(2500) for _ in range(n)]
    lq = [pick(200) for _ in range(n)]
    lk = [max(0, x + rng.randint(-50, 300)) for x in lq]
    return lq, lk


def _forward_case(i):
    rng = random.Random(91000 + i)
    path = rng.choice(["packed", "paged", "fp8", "paged_fp8"])
    fp8 = path in ("fp8", "paged_fp8")
    D = 128 if fp8 else rng.choice([64, 128])
    dtype = rng.choice(["fp16", "bf16"])
    Hkv = rng.choice([1, 2, 4, 8])
    group = rng.choice([1, 2, 3, 4, 8, 16, 20] if Hkv <= 2 else [1, 2, 4])
    kind = rng.choice(["prefill", "decode", "mixed"])
    lq, lk = _lengths(rng, kind)
    if sum(lq) == 0:
        lq[0] = 1
        lk[0] = max(lk[0], 1)
    cfg = dict(path=path, kind=kind, seqlens_q=lq, seqlens_k=lk, Hq=Hkv * group, Hkv=Hkv, D=D, dtype=dtype,
               causal=rng.random() < 0.6, alibi=rng.random() < 0.4,
               page_size=rng.choice([64, 128, 192, 256]))
    return cfg


def _run_paged(inp, page_size, seed):
    from memory_efficient_attention_amd import attention_paged
    pk = to_paged(inp, page_size, seed=seed)
    dev = "cuda"
    out = torch.full(tuple(inp.q.shape), float("nan"), dtype=inp.q.dtype, device=dev)
    res = attention_paged(inp.q.to(dev), pk.k_cache.to(dev), pk.v_cache.to(dev), pk.block_table.to(dev),
                          inp.seqstart_q.to(dev), inp.seqstart_k.to(dev), inp.max_seqlen_q, inp.max_seqlen_k,
                          causal=inp.causal,
                          alibi_slopes=None if inp.alibi_slopes is None else inp.alibi_slopes.to(dev),
                          scale=inp.scale, return_lse=True, out=out, total_k=inp.total_k)
    torch.cuda.synchronize()
    return res[0].cpu(), res[1].cpu()


def _run_fp8(inp, f, page_size, seed, out_dtype):
    from memory_efficient_attention_amd import attention_packed_fp8, attention_paged_fp8
    dev = "cuda"
    out = torch.full(tuple(inp.q.shape), float("nan"), dtype=out_dtype, device=dev)
    slopes = None if inp.alibi_slopes is None else inp.alibi_slopes.to(dev)
    common = dict(causal=inp.causal, alibi_slopes=slopes, scale=inp.scale, out_dtype=out_dtype, return_lse=True,
                  out=out)
    if page_size is None:
        res = attention_packed_fp8(f.q8.to(dev), f.k8.to(dev), f.v8.to(dev), f.q_scale, f.k_scale, f.v_scale,
                                   inp.seqstart_q.to(dev), inp.seqstart_k.to(dev), inp.max_seqlen_q,
                                   inp.max_seqlen_k, **common)
    else:
        pk = to_paged(dataclasses.replace(inp, k=f.k8, v=f.v8), page_size, seed=seed)
        res = attention_paged_fp8(f.q8.to(dev), pk.k_cache.to(dev), pk.v_cache.to(dev), f.q_scale, f.k_scale,
                                  f.v_scale, pk.block_table.to(dev), inp.seqstart_q.to(dev),
                                  inp.seqstart_k.to(dev), inp.max_seqlen_q, inp.max_seqlen_k,
                                  total_k=inp.total_k, **common)
    torch.cuda.synchronize()
    return res[0].cpu(), res[1].cpu()


@pytest.mark.parametrize("i", range(N_FORWARD))
def test_forward_sweep(i):
    cfg = _forward_case(i)
    _log(f"sweep forward {i}: {cfg}")
    inp = random_case(92000 + i, cfg["seqlens_q"], cfg["seqlens_k"], Hq=cfg["Hq"], Hkv=cfg["Hkv"], D=cfg["D"],
                      dtype=cfg["dtype"], causal=cfg["causal"], alibi=cfg["alibi"])
    path = cfg["path"]
    if path in ("fp8", "paged_fp8"):
        out_dtype = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float16
        f = to_fp8(inp)
        out, lse = _run_fp8(inp, f, cfg["page_size"] if path == "paged_fp8" else None, i, out_dtype)
        ref_out, ref_lse = oracle.attention_forward_fp8(f.q8, f.k8, f.v8, f.q_scale, f.k_scale, f.v_scale,
                                                        inp.seqstart_q, inp.seqstart_k, causal=inp.causal,
                                                        alibi_slopes=inp.alibi_slopes, scale=inp.scale)
    else:
        out, lse = _run_paged(inp, cfg["page_size"], i) if path == "paged" else run_gpu(inp)
        ref_out, ref_lse = oracle_full(inp)
    _log(f"  {compare(out, lse, ref_out, ref_lse, cfg['dtype'], f'sweep forward {i}')}")


def _backward_case(i):
    rng = random.Random(93000 + i)
    Hkv = rng.choice([1, 2, 4])
    kind = rng.choice(["prefill", "mixed"])
    lq, lk = _lengths(rng, kind)
    if sum(lq) == 0:
        lq[0] = 1
        lk[0] = max(lk[0], 1)
    return dict(kind=kind, seqlens_q=lq, seqlens_k=lk, Hq=Hkv * rng.choice([1, 2, 4]), Hkv=Hkv,
                D=rng.choice([64, 128]), dtype=rng.choice(["fp16", "bf16"]), causal=rng.random() < 0.6,
                alibi=rng.random() < 0.4)


@pytest.mark.parametrize("i", range(N_BACKWARD))
def test_backward_sweep(i):
    cfg = _backward_case(i)
    _log(f"sweep backward {i}: {cfg}")
    inp = random_case(94000 + i, cfg["seqlens_q"], cfg["seqlens_k"], Hq=cfg["Hq"], Hkv=cfg["Hkv"], D=cfg["D"],
                      dtype=cfg["dtype"], causal=cfg["causal"], alibi=cfg["alibi"])
    dout = random_dout(94000 + i, inp)
    got = run_gpu_backward(inp, dout)
    ref = oracle_backward(inp, dout)
    _log(f"  {compare_grads(got, ref, cfg['dtype'], f'sweep backward {i}')}")
