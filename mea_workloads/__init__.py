"""Seeded synthetic inputs for the attention-forward workloads.

This module is shared by the tests, the benchmark and the oracle side. It holds
none of the attention arithmetic: only how sequence lengths, q/k/v and the
per-head ALiBi slopes (which callers pass in as an input) are drawn.

Recipe (the same for every workload):
  * lengths: ``numpy.random.default_rng(seed).integers(lo, hi, size=n,
    endpoint=True)``;
  * tensors: one ``torch.Generator('cpu').manual_seed(seed + 1)``, then
    ``torch.randn(shape, dtype=float32)`` for q, k and v in that order, then a
    cast to the workload's dtype (round to nearest even).  Everything is drawn
    on the host, so a device copy and the oracle see identical bits;
  * ALiBi slopes: ``2 ** (-8 (h + 1) / Hq)`` per query head, evaluated in
    float64 and rounded to float32.

Layouts are packed and row-major: q ``[Tq, Hq, D]``, k and v ``[Tk, Hkv, D]``,
``seqstart_q`` / ``seqstart_k`` int32 ``[n + 1]``.  Query head ``h`` reads
key/value head ``h // (Hq // Hkv)``.  A BMGHK tensor ``[B, M, G, Hq', K]``
(the grouped-query layout of the xFormers tutorial page, section 5) is the same
memory viewed as ``[B*M, G*Hq', K]``, so the BMGHK workload is generated in
that shape and viewed packed.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

__all__ = [
    "Workload", "Inputs", "WORKLOADS", "get_workload", "generate", "random_case",
    "alibi_slopes", "seqstart_from_lengths", "sample_rows", "prefix", "PagedKV", "to_paged",
    "random_dout", "Fp8Inputs", "to_fp8", "FfnInputs", "swiglu_case", "FFN_WORKLOAD", "mixed_case",
    "MIXED_WORKLOAD",
]

_DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One named workload: shapes, dtype, mask kind and how lengths are drawn."""

    name: str
    description: str
    dtype: str                      # "fp16" | "bf16"
    Hq: int
    Hkv: int
    D: int
    causal: bool
    alibi: bool
    # exactly one of the following length recipes is used
    seqlens: Optional[Tuple[int, ...]] = None        # fixed q = k lengths
    num_seqs: int = 0                                # random lengths ...
    len_lo: int = 0
    len_hi: int = 0
    decode: bool = False            # q length 1 per request, k length random
    bmghk: Optional[Tuple[int, int, int, int]] = None  # (B, M, G, Hq per group)


WORKLOADS = {
    w.name: w
    for w in [
        Workload(
            name="packed_varlen_h8_d64_fp16",
            description="packed varlen [37,120,8,200], 8 q/kv heads, D=64, fp16",
            dtype="fp16", Hq=8, Hkv=8, D=64, causal=False, alibi=False,
            seqlens=(37, 120, 8, 200)),
        Workload(
            name="bmghk_gqa_b2_m256_g2x4_d64_fp16",
            description="BMGHK B=2 M=256 G=2 groups x 4 q heads, D=64, fp16, no mask",
            dtype="fp16", Hq=8, Hkv=2, D=64, causal=False, alibi=False,
            seqlens=(256, 256), bmghk=(2, 256, 2, 4)),
        Workload(
            name="causal_alibi_gqa_4x2048_h32kv8_d128_bf16",
            description="4 x 2048 tokens, 32 q / 8 kv heads, D=128, bf16, causal + ALiBi",
            dtype="bf16", Hq=32, Hkv=8, D=128, causal=True, alibi=True,
            seqlens=(2048, 2048, 2048, 2048)),
        Workload(
            name="varlen_causal_gqa_64seq_h32kv8_d128_bf16",
            description="64 packed sequences, lengths U[128,4096], 32 q / 8 kv heads, "
                        "D=128, bf16, block-diagonal causal",
            dtype="bf16", Hq=32, Hkv=8, D=128, causal=True, alibi=False,
            num_seqs=64, len_lo=128, len_hi=4096),
        Workload(
            name="decode_splitkv_64req_h64kv8_d128_bf16",
            description="64 requests x 1 query, KV lengths U[1024,32768], 64 q / 8 kv "
                        "heads, D=128, bf16, split-KV + LSE combine",
            dtype="bf16", Hq=64, Hkv=8, D=128, causal=False, alibi=False,
            num_seqs=64, len_lo=1024, len_hi=32768, decode=True),
    ]
}


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None


@dataclasses.dataclass
class Inputs:
    """Host tensors for one call.  ``scale`` is a float32-representable float."""

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    seqstart_q: torch.Tensor        # int32 [n+1]
    seqstart_k: torch.Tensor        # int32 [n+1]
    seqlens_q: List[int]
    seqlens_k: List[int]
    Hq: int
    Hkv: int
    D: int
    causal: bool
    alibi_slopes: Optional[torch.Tensor]   # float32 [Hq] or None
    scale: float
    dtype: str
    bmghk: Optional[Tuple[int, int, int, int]] = None

    @property
    def total_q(self) -> int:
        return int(self.seqstart_q[-1])

    @property
    def total_k(self) -> int:
        return int(self.seqstart_k[-1])

    @property
    def max_seqlen_q(self) -> int:
        return max(self.seqlens_q) if self.seqlens_q else 0

    @property
    def max_seqlen_k(self) -> int:
        return max(self.seqlens_k) if self.seqlens_k else 0


def alibi_slopes(Hq: int) -> torch.Tensor:
    """Per-query-head ALiBi slopes 2^(-8(h+1)/Hq), float64 rounded to float32."""
    vals = [2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)]
    return torch.tensor(vals, dtype=torch.float64).to(torch.float32)


def default_scale(D: int) -> float:
    """1/sqrt(D) rounded to float32 (the value the C entry point receives)."""
    return float(np.float32(1.0 / math.sqrt(D)))


def seqstart_from_lengths(lengths: Sequence[int]) -> torch.Tensor:
    out = [0]
    for L in lengths:
        out.append(out[-1] + int(L))
    return torch.tensor(out, dtype=torch.int32)


def _lengths(w: Workload, seed: int) -> Tuple[List[int], List[int]]:
    if w.seqlens is not None:
        return list(w.seqlens), list(w.seqlens)
    rng = np.random.default_rng(seed)
    lk = [int(x) for x in rng.integers(w.len_lo, w.len_hi, size=w.num_seqs, endpoint=True)]
    if w.decode:
        return [1] * w.num_seqs, lk
    return lk, list(lk)


def _randn(g: torch.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)


def generate(name_or_workload, seed: int = 0, *, causal: Optional[bool] = None,
             alibi: Optional[bool] = None, num_seqs: Optional[int] = None) -> Inputs:
    """Draw the inputs of one workload.

    ``causal`` / ``alibi`` override the workload's mask choice (the pages run
    the packed workload once without and once with the causal mask, and the
    long varlen workload with and without ALiBi).  ``num_seqs`` keeps only the
    first ``num_seqs`` sequences of a random-length workload (the same lengths
    the full workload draws; the tensors are then drawn for that prefix only).
    """
    w = name_or_workload if isinstance(name_or_workload, Workload) else get_workload(name_or_workload)
    lq, lk = _lengths(w, seed)
    if num_seqs is not None:
        lq, lk = lq[:num_seqs], lk[:num_seqs]
    dt = _DTYPES[w.dtype]
    g = torch.Generator("cpu").manual_seed(seed + 1)
    Tq, Tk = sum(lq), sum(lk)
    if w.bmghk is not None and num_seqs is None:
        B, M, G, Hg = w.bmghk
        q = _randn(g, (B, M, G, Hg, w.D), dt).view(B * M, G * Hg, w.D)
        k = _randn(g, (B, M, G, 1, w.D), dt).view(B * M, G, w.D)
        v = _randn(g, (B, M, G, 1, w.D), dt).view(B * M, G, w.D)
    else:
        q = _randn(g, (Tq, w.Hq, w.D), dt)
        k = _randn(g, (Tk, w.Hkv, w.D), dt)
        v = _randn(g, (Tk, w.Hkv, w.D), dt)
    use_causal = w.causal if causal is None else causal
    use_alibi = w.alibi if alibi is None else alibi
    return Inputs(
        q=q, k=k, v=v,
        seqstart_q=seqstart_from_lengths(lq), seqstart_k=seqstart_from_lengths(lk),
        seqlens_q=lq, seqlens_k=lk, Hq=w.Hq, Hkv=w.Hkv, D=w.D,
        causal=use_causal, alibi_slopes=alibi_slopes(w.Hq) if use_alibi else None,
        scale=default_scale(w.D), dtype=w.dtype, bmghk=w.bmghk if num_seqs is None else None)


def random_case(seed: int, seqlens_q: Sequence[int], seqlens_k: Optional[Sequence[int]] = None,
                Hq: int = 4, Hkv: int = 2, D: int = 64, dtype: str = "fp16",
                causal: bool = False, alibi: bool = False, scale: Optional[float] = None,
                slopes: Optional[torch.Tensor] = None, std: float = 1.0) -> Inputs:
    """A free-form case for parity tests: given lengths, random N(0, std^2) q/k/v."""
    lq = [int(x) for x in seqlens_q]
    lk = list(lq) if seqlens_k is None else [int(x) for x in seqlens_k]
    assert len(lq) == len(lk)
    dt = _DTYPES[dtype] if isinstance(dtype, str) else dtype
    g = torch.Generator("cpu").manual_seed(seed + 1)
    Tq, Tk = sum(lq), sum(lk)
    q = (torch.randn((Tq, Hq, D), generator=g) * std).to(dt)
    k = (torch.randn((Tk, Hkv, D), generator=g) * std).to(dt)
    v = (torch.randn((Tk, Hkv, D), generator=g) * std).to(dt)
    if alibi and slopes is None:
        slopes = alibi_slopes(Hq)
    return Inputs(
        q=q, k=k, v=v,
        seqstart_q=seqstart_from_lengths(lq), seqstart_k=seqstart_from_lengths(lk),
        seqlens_q=lq, seqlens_k=lk, Hq=Hq, Hkv=Hkv, D=D, causal=causal,
        alibi_slopes=slopes if alibi else None,
        scale=default_scale(D) if scale is None else float(np.float32(scale)),
        dtype=dtype if isinstance(dtype, str) else {v_: k_ for k_, v_ in _DTYPES.items()}[dt])


MIXED_WORKLOAD = dict(prefills=8, prefill_lo=128, prefill_hi=4096, decodes=56, decode_lo=1024, decode_hi=32768,
                      Hq=32, Hkv=8, D=128, dtype="bf16")


def mixed_case(seed: int = 0, prefills: int = 8, decodes: int = 56, prefill_lo: int = 128, prefill_hi: int = 4096,
               decode_lo: int = 1024, decode_hi: int = 32768, Hq: int = 32, Hkv: int = 8, D: int = 128,
               dtype: str = "bf16", causal: bool = True, alibi: bool = False) -> Inputs:
    """A serving engine's mixed batch: ``prefills`` prompts with lengths
    U[prefill_lo, prefill_hi] (queries = keys), then ``decodes`` decode steps
    of one query each over KV histories of lengths U[decode_lo, decode_hi];
    lengths from ``numpy.random.default_rng(seed)`` (prefills first), tensors
    as for every workload."""
    rng = np.random.default_rng(seed)
    pre = [int(x) for x in rng.integers(prefill_lo, prefill_hi, size=prefills, endpoint=True)]
    dec = [int(x) for x in rng.integers(decode_lo, decode_hi, size=decodes, endpoint=True)]
    return random_case(seed, pre + [1] * decodes, pre + dec, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, causal=causal,
                       alibi=alibi)


def random_dout(seed: int, inp: Inputs, std: float = 1.0) -> torch.Tensor:
    """A seeded upstream gradient dO for ``inp``: N(0, std^2) of q's shape and dtype."""
    g = torch.Generator("cpu").manual_seed(seed + 7919)
    return (torch.randn(tuple(inp.q.shape), generator=g) * std).to(inp.q.dtype)


def prefix(inp: Inputs, n: int) -> Inputs:
    """The first ``n`` sequences of ``inp`` as views of the same tensors (the
    rows a call on the whole of ``inp`` produces for them are comparable)."""
    sq, sk = inp.seqstart_q.tolist(), inp.seqstart_k.tolist()
    return dataclasses.replace(
        inp, q=inp.q[:sq[n]], k=inp.k[:sk[n]], v=inp.v[:sk[n]],
        seqstart_q=inp.seqstart_q[:n + 1].clone(), seqstart_k=inp.seqstart_k[:n + 1].clone(),
        seqlens_q=inp.seqlens_q[:n], seqlens_k=inp.seqlens_k[:n], bmghk=None)


FP8_MAX = 448.0   # largest finite OCP e4m3 value


@dataclasses.dataclass
class Fp8Inputs:
    """q, k, v of an input quantised to OCP e4m3 with one float32 scale per
    tensor: the values meant are scale * tensor."""
    q8: torch.Tensor           # float8_e4m3fn [Tq, Hq, D]
    k8: torch.Tensor           # float8_e4m3fn [Tk, Hkv, D]
    v8: torch.Tensor           # float8_e4m3fn [Tk, Hkv, D]
    q_scale: float
    k_scale: float
    v_scale: float


def _quantise(x: torch.Tensor) -> Tuple[torch.Tensor, float]:
    """Per-tensor scale max|x| / 448 (float32), values x / scale rounded to e4m3."""
    amax = float(x.float().abs().max()) if x.numel() else 0.0
    scale = float(np.float32(amax / FP8_MAX)) if amax > 0 else 1.0
    return (x.float() / scale).to(torch.float8_e4m3fn), scale


def to_fp8(inp: Inputs) -> Fp8Inputs:
    """The q, k, v of ``inp`` quantised to e4m3 with per-tensor scales (the
    rest of ``inp`` -- lengths, masks, slopes, score scale -- applies as is)."""
    q8, qs = _quantise(inp.q)
    k8, ks = _quantise(inp.k)
    v8, vs = _quantise(inp.v)
    return Fp8Inputs(q8=q8, k8=k8, v8=v8, q_scale=qs, k_scale=ks, v_scale=vs)


@dataclasses.dataclass
class FfnInputs:
    """Inputs of one SwiGLU feed-forward call (host tensors)."""
    x: torch.Tensor        # [tokens, d_model]
    w_gate: torch.Tensor   # [d_ff, d_model]
    w_up: torch.Tensor     # [d_ff, d_model]
    w_down: torch.Tensor   # [d_model, d_ff]
    dtype: str


# The feed-forward layer of the prefill workload's transformer block: its
# 137,663 packed tokens, d_model = 32 heads x 128, d_ff = 11008 (the LLaMA-7B
# feed-forward width; the zizhi168.cn page uses LLaMA-7B as its example model).
FFN_WORKLOAD = dict(tokens=137663, d_model=4096, d_ff=11008, dtype="bf16")


def swiglu_case(seed: int, tokens: int, d_model: int, d_ff: int, dtype: str = "bf16") -> FfnInputs:
    """x ~ N(0, 1); weights ~ N(0, 1 / fan_in), so that activations stay O(1)."""
    dt = _DTYPES[dtype]
    g = torch.Generator("cpu").manual_seed(seed + 11)
    x = torch.randn((tokens, d_model), generator=g).to(dt)
    w_gate = (torch.randn((d_ff, d_model), generator=g) * d_model ** -0.5).to(dt)
    w_up = (torch.randn((d_ff, d_model), generator=g) * d_model ** -0.5).to(dt)
    w_down = (torch.randn((d_model, d_ff), generator=g) * d_ff ** -0.5).to(dt)
    return FfnInputs(x=x, w_gate=w_gate, w_up=w_up, w_down=w_down, dtype=dtype)


@dataclasses.dataclass
class PagedKV:
    """K/V of a packed input scattered into a paged cache."""
    k_cache: torch.Tensor      # [num_pages, page_size, Hkv, D]
    v_cache: torch.Tensor      # [num_pages, page_size, Hkv, D]
    block_table: torch.Tensor  # int32 [num_seqs, max_blocks]
    page_size: int


def to_paged(inp: Inputs, page_size: int, seed: int = 0, spare_pages: int = 3,
             filler: float = float("nan")) -> PagedKV:
    """Scatter the keys and values of ``inp`` into pages of ``page_size`` keys
    in a seeded random page order, with ``spare_pages`` unused pages.  Every
    slot that holds no key of a sequence (the tail of a sequence's last page,
    the spare pages) is set to ``filler``, so a read of such a slot shows up in
    the result.  Unused block-table entries point at page 0."""
    lens = list(inp.seqlens_k)
    blocks = [-(-L // page_size) for L in lens]
    num_pages = sum(blocks) + spare_pages
    max_blocks = max([1] + blocks)
    perm = np.random.default_rng(seed + 777).permutation(num_pages)
    shape = (num_pages, page_size, inp.Hkv, inp.D)
    k_cache = torch.full(shape, filler, dtype=inp.k.dtype)
    v_cache = torch.full(shape, filler, dtype=inp.v.dtype)
    table = torch.zeros((len(lens), max_blocks), dtype=torch.int32)
    sk = inp.seqstart_k.tolist()
    nxt = 0
    for b, L in enumerate(lens):
        for i in range(blocks[b]):
            page = int(perm[nxt])
            nxt += 1
            table[b, i] = page
            j0, j1 = i * page_size, min(L, (i + 1) * page_size)
            k_cache[page, :j1 - j0] = inp.k[sk[b] + j0:sk[b] + j1]
            v_cache[page, :j1 - j0] = inp.v[sk[b] + j0:sk[b] + j1]
    return PagedKV(k_cache, v_cache, table, page_size)


def sample_rows(inp: Inputs, count: int, seed: int = 0) -> List[Tuple[int, int]]:
    """Deterministic (token, q head) picks for sampled checks at full size.

    Always includes the first and last token of the first and last non-empty
    sequence (the edges of the packing) and the last token of the longest one.
    """
    rng = np.random.default_rng(seed + 12345)
    picks = set()
    nonempty = [b for b, L in enumerate(inp.seqlens_q) if L > 0]
    sq = inp.seqstart_q.tolist()
    if nonempty:
        longest = max(nonempty, key=lambda b: inp.seqlens_q[b])
        for b in (nonempty[0], nonempty[-1], longest):
            picks.add((sq[b], 0))
            picks.add((sq[b + 1] - 1, inp.Hq - 1))
    Tq = inp.total_q
    while len(picks) < count and Tq > 0:
        picks.add((int(rng.integers(0, Tq)), int(rng.integers(0, inp.Hq))))
    return sorted(picks)
