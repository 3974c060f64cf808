"""GPU parity of the fp8 forward (``mea_fwd_fp8``): q, k, v quantised to OCP
e4m3 with per-tensor scales; the HIP result is compared with the float64
oracle on the same codes and scales (``attention_forward_fp8``), with the
output gates of the 16-bit path for the output dtype."""
import dataclasses
import sys

import pytest
import torch

import oracle
from mea_workloads import generate, random_case, sample_rows, to_fp8
from parity import compare

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _run(inp, f, out_dtype):
    from memory_efficient_attention_amd import attention_packed_fp8
    dev = "cuda"
    out = torch.full((inp.total_q, inp.Hq, inp.D), float("nan"), dtype=out_dtype, device=dev)
    res = attention_packed_fp8(f.q8.to(dev), f.k8.to(dev), f.v8.to(dev), f.q_scale, f.k_scale, f.v_scale,
                               inp.seqstart_q.to(dev), inp.seqstart_k.to(dev), inp.max_seqlen_q, inp.max_seqlen_k,
                               causal=inp.causal,
                               alibi_slopes=None if inp.alibi_slopes is None else inp.alibi_slopes.to(dev),
                               scale=inp.scale, out_dtype=out_dtype, return_lse=True, out=out)
    torch.cuda.synchronize()
    return res[0].cpu(), res[1].cpu()


def _ref(inp, f):
    return oracle.attention_forward_fp8(f.q8, f.k8, f.v8, f.q_scale, f.k_scale, f.v_scale, inp.seqstart_q,
                                        inp.seqstart_k, causal=inp.causal, alibi_slopes=inp.alibi_slopes,
                                        scale=inp.scale)


CASES = [
    # (name, seqlens_q, seqlens_k, Hq, Hkv, causal, alibi, out dtype)
    ("varlen_causal_bf16", [37, 120, 8, 200], None, 8, 8, True, False, torch.bfloat16),
    ("varlen_alibi_fp16", [37, 120, 8, 200], None, 8, 8, False, True, torch.float16),
    ("gqa_causal_alibi", [130, 1, 77, 300], None, 8, 2, True, True, torch.bfloat16),
    ("mqa", [256, 129], None, 8, 1, False, False, torch.float16),
    ("lq_gt_lk_causal", [3, 5, 70, 150], [7, 2, 200, 64], 4, 2, True, False, torch.bfloat16),
    ("lq_lt_lk_causal_alibi", [65, 17, 200], [300, 17, 333], 4, 4, True, True, torch.bfloat16),
    ("empty_sides", [0, 65, 10, 0, 33], [5, 0, 10, 0, 129], 4, 2, True, False, torch.bfloat16),
    # decode-shaped calls (max_seqlen_q == 1) take the split-KV decode kernels
    ("decode_gqa_alibi", [1, 1, 1, 1], [300, 1, 64, 1000], 8, 2, True, True, torch.bfloat16),
    ("decode_group8_long", [1] * 6, [5000, 33, 1, 4097, 64, 129], 64, 8, True, False, torch.bfloat16),
    ("decode_mqa_alibi_fp16", [1, 1, 1], [2000, 65, 700], 16, 1, True, True, torch.float16),
    ("decode_group20", [1, 1, 1, 1, 1], [1, 130, 0, 3000, 257], 40, 2, True, False, torch.bfloat16),
    ("decode_empty_rows", [1, 0, 1], [0, 5, 64], 8, 8, True, False, torch.bfloat16),
    ("decode_tails", [1] * 7, [31, 32, 33, 63, 64, 65, 97], 8, 4, True, True, torch.bfloat16),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_fp8_parity(ci):
    name, lq, lk, Hq, Hkv, causal, alibi, odt = CASES[ci]
    inp = random_case(700 + ci, lq, lk, Hq=Hq, Hkv=Hkv, D=128, dtype="bf16", causal=causal, alibi=alibi)
    f = to_fp8(inp)
    _log(f"fp8 {name}")
    out, lse = _run(inp, f, odt)
    ref_out, ref_lse = _ref(inp, f)
    _log(f"  {compare(out, lse, ref_out, ref_lse, 'bf16' if odt == torch.bfloat16 else 'fp16', name)}")


def test_fp8_causal_alibi_gqa_4x2048():
    inp = generate("causal_alibi_gqa_4x2048_h32kv8_d128_bf16")
    f = to_fp8(inp)
    _log("fp8 4x2048")
    out, lse = _run(inp, f, torch.bfloat16)
    ref_out, ref_lse = _ref(inp, f)
    _log(f"  {compare(out, lse, ref_out, ref_lse, 'bf16', 'fp8 4x2048')}")


def test_fp8_full_size_sampled():
    """The 64-sequence prefill workload (137,663 tokens) in fp8; sampled rows."""
    inp = generate("varlen_causal_gqa_64seq_h32kv8_d128_bf16")
    f = to_fp8(inp)
    _log("fp8 full size")
    out, lse = _run(inp, f, torch.bfloat16)
    assert not torch.isnan(out).any()
    rows = sample_rows(inp, 160, seed=5)
    q = f.q8.to(torch.float64) * f.q_scale
    k = f.k8.to(torch.float64) * f.k_scale
    v = f.v8.to(torch.float64) * f.v_scale
    ro, rl = oracle.attention_rows(q, k, v, inp.seqstart_q, inp.seqstart_k, rows, causal=True,
                                   scale=inp.scale)
    go = torch.stack([out[t, h] for t, h in rows])
    gl = torch.stack([lse[h, t] for t, h in rows])
    _log(f"  {compare(go, gl, ro, rl, 'bf16', 'fp8 full size sampled')}")


def test_fp8_decode_full_size_sampled():
    """The 64-request decode workload (1.1 M KV tokens, Hq 64 / Hkv 8) in fp8;
    sampled rows against the oracle on the dequantised values."""
    inp = generate("decode_splitkv_64req_h64kv8_d128_bf16")
    f = to_fp8(inp)
    _log(f"fp8 decode full size, sum Lk={inp.total_k}")
    out, lse = _run(inp, f, torch.bfloat16)
    assert not torch.isnan(out).any()
    rows = sample_rows(inp, 128, seed=9)
    q = f.q8.to(torch.float64) * f.q_scale
    k = f.k8.to(torch.float64) * f.k_scale
    v = f.v8.to(torch.float64) * f.v_scale
    ro, rl = oracle.attention_rows(q, k, v, inp.seqstart_q, inp.seqstart_k, rows, causal=inp.causal,
                                   scale=inp.scale)
    go = torch.stack([out[t, h] for t, h in rows])
    gl = torch.stack([lse[h, t] for t, h in rows])
    _log(f"  {compare(go, gl, ro, rl, 'bf16', 'fp8 decode sampled')}")


def test_fp8_decode_matches_prefill_kernel_rows():
    """A decode row is also the last row of a prefill-shaped call over the
    same keys: with a second query row added to every sequence the call takes
    the prefill kernel, and its last rows must agree with the decode kernel's
    to the output tolerance (both are checked against the oracle above; this
    ties the two fp8 paths to each other on the same codes)."""
    lk = [300, 1, 64, 1000, 4097]
    inp = random_case(790, [1] * len(lk), lk, Hq=16, Hkv=4, D=128, dtype="bf16", causal=True)
    f = to_fp8(inp)
    out_d, lse_d = _run(inp, f, torch.bfloat16)
    # prefill-shaped: each sequence gets its decode query as its last of two rows
    inp2 = random_case(790, [2] * len(lk), lk, Hq=16, Hkv=4, D=128, dtype="bf16", causal=True)
    f2 = to_fp8(inp2)
    q8 = f2.q8.clone()
    q8[1::2] = f.q8
    f2 = dataclasses.replace(f2, q8=q8, k8=f.k8, v8=f.v8, q_scale=f.q_scale, k_scale=f.k_scale, v_scale=f.v_scale)
    out_p, lse_p = _run(inp2, f2, torch.bfloat16)
    d_out = (out_d.double() - out_p[1::2].double()).abs().max().item()
    d_lse = (lse_d.double() - lse_p[:, 1::2].double()).abs().max().item()
    _log(f"  decode vs prefill kernel: out {d_out:.2e}, lse {d_lse:.2e}")
    assert d_out <= 1e-2 and d_lse <= 1e-3


def test_fp8_decode_wide_head_groups():
    """Decode with 8 key/value heads and over half a million keys, so that the
    pieces stay at least 2048 keys long and each fp8 decode workgroup takes
    all 8 heads of a token row.  Every row is checked against the oracle, one
    key/value head (and its two query heads) at a time, so that the oracle
    holds one head's keys in float64; a second call must give the same bits."""
    lk = [0, 1, 31, 33, 2047, 2049, 100000, 65, 250000, 4097, 200000, 129]
    inp = random_case(797, [1] * len(lk), lk, Hq=16, Hkv=8, D=128, dtype="bf16", causal=True, alibi=True)
    f = to_fp8(inp)
    _log(f"fp8 decode, 8-head groups: {len(lk)} requests, sum Lk={inp.total_k}, Hq 16 / Hkv 8")
    out, lse = _run(inp, f, torch.bfloat16)
    out2, lse2 = _run(inp, f, torch.bfloat16)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    for g in range(8):
        hs = [2 * g, 2 * g + 1]
        q = f.q8[:, hs].to(torch.float64) * f.q_scale
        k = f.k8[:, [g]].to(torch.float64) * f.k_scale
        v = f.v8[:, [g]].to(torch.float64) * f.v_scale
        rows = [(t, j) for t in range(inp.total_q) for j in range(2)]
        ro, rl = oracle.attention_rows(q, k, v, inp.seqstart_q, inp.seqstart_k, rows, causal=True,
                                       alibi_slopes=inp.alibi_slopes[hs], scale=inp.scale)
        go = torch.stack([out[t, hs[j]] for t, j in rows])
        gl = torch.stack([lse[hs[j], t] for t, j in rows])
        _log(f"  {compare(go, gl, ro, rl, 'bf16', f'8-head groups, key/value head {g}')}")


def test_fp8_decode_deterministic():
    inp = random_case(795, [1] * 6, [5000, 33, 1, 4097, 64, 129], Hq=64, Hkv=8, D=128, dtype="bf16", causal=True)
    f = to_fp8(inp)
    o1, l1 = _run(inp, f, torch.bfloat16)
    for _ in range(3):
        o2, l2 = _run(inp, f, torch.bfloat16)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
