#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic inputs:
  1. packed causal GQA prefill: 64 sequences with lengths U[128, 4096] from
     seed 0 (137,663 tokens), 32 query / 8 key-value heads, D = 128, bf16,
     block-diagonal causal mask, no ALiBi;
  2. split-KV decode: 64 requests x 1 query, KV lengths U[1024, 32768] from
     seed 0 (1,101,299 KV tokens), 64 query / 8 key-value heads, D = 128, bf16,
     partial kernel + log-sum-exp combine.
Inputs are drawn on the host and copied to HBM before the timed region.

Prints one JSON line.  ``value`` is the prefill throughput in TFLOP/s counting
only unmasked score FLOPs (4 * D per allowed (query, key, head) triple) over
the prefill kernel's own time (HIP events on its launch stream); the decode
figures (GB/s of algorithmic bytes Q + K + V + O + LSE) are in ``decode``.
``roofline`` describes the prefill kernel against the bf16 dense MFMA peak,
``decode.roofline`` the decode launches against HBM bandwidth, and
``cpu_baseline`` times the CPU float64 oracle on a bounded sample of the
prefill workload.  Outside the step, ``prefill_alibi`` times the prefill
workload with ALiBi, ``decode_paged`` the decode workload with K/V in a
paged cache (pages of 64 keys in a shuffled order, through mea_fwd_paged),
``backward`` the prefill workload's gradients (mea_bwd, dq/dk/dv from a
seeded dO) at 2.5x the forward's unmasked FLOPs (five products against two),
``prefill_fp8`` the prefill workload with q, k, v quantised to OCP e4m3
(mea_fwd_fp8, per-tensor scales, bf16 output), ``decode_fp8`` and
``decode_paged_fp8`` the decode workload quantised the same way (packed, and
in the shuffled 64-key pages through mea_fwd_paged_fp8), ``swiglu_ffn`` the SwiGLU
feed-forward layer of the same block on the same 137,663 tokens (d_model
4096, d_ff 11008, bf16; 6 * T * d_model * d_ff FLOPs), ``prefill_4x2048``
the 4 x 2048-token causal ALiBi GQA prefill (32 query / 8 key-value heads,
D = 128, bf16) with its own roofline, and ``mixed`` a serving engine's mixed
batch (8 prefills U[128, 4096] then 56 decode steps over U[1024, 32768]
keys, 32/8 heads) through mea_fwd_mixed, with its prefill part (TFLOP/s) and
decode part (GB/s) timed on their own and the whole batch through the
prefill kernels for comparison.  ``cpu_baseline`` also times the oracle
on samples of the decode workload and on the small parity workloads, and
records the host's CPU model and core count.

``python bench.py --write-traffic DIR`` turns rocprofv3 FETCH_SIZE /
WRITE_SIZE counter runs of the parts (``DIR/pmc_<part>_<COUNTER>/``, one
counter per run, the ``copy`` part included for calibration) into
profiles/hbm_traffic.json, keyed by the kernel-source hash.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (% MFMA peak) packed causal GQA; decode GB/s (% HBM)"
PEAK_MFMA_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0            # HBM3E
PREFILL = "varlen_causal_gqa_64seq_h32kv8_d128_bf16"
DECODE = "decode_splitkv_64req_h64kv8_d128_bf16"
PREFILL_4X2048 = "causal_alibi_gqa_4x2048_h32kv8_d128_bf16"
SMALL_WORKLOADS = ["packed_varlen_h8_d64_fp16", "bmghk_gqa_b2_m256_g2x4_d64_fp16"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = ["fwd_prefill.hip", "fwd_decode.hip", "bwd.hip", "ffn.hip", "mea_common.h", "mea_launch.h",
                  "mea_tiles.h"]


def unmasked_flops(inp) -> int:
    """4*D FLOPs per allowed (query row, key, query head) triple."""
    total = 0
    for Lq, Lk in zip(inp.seqlens_q, inp.seqlens_k):
        if inp.causal:
            off = Lk - Lq
            pairs = sum(max(0, min(Lk, r + off + 1)) for r in range(Lq)) if Lq != Lk else Lq * (Lq + 1) // 2
        else:
            pairs = Lq * Lk
        total += pairs
    return 4 * inp.D * inp.Hq * total


def algorithmic_bytes(inp, with_lse=True) -> int:
    """Q + K + V + O (+ LSE): every input byte read once, every output written once."""
    b = 2 * (inp.q.numel() * 2 + inp.k.numel() + inp.v.numel())
    if with_lse:
        b += inp.Hq * inp.total_q * 4
    return b


def algorithmic_bytes_fp8(inp, with_lse=True) -> int:
    """The fp8 call's Q + K + V (one byte each) + O (bf16) (+ LSE)."""
    b = inp.q.numel() * (1 + 2) + inp.k.numel() + inp.v.numel()
    if with_lse:
        b += inp.Hq * inp.total_q * 4
    return b


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: comments and blank space are dropped
    first, so that an edit of a comment does not orphan the counter runs."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "memory_efficient_attention_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("kernels", {}).get(kernel)


class Call:
    """Pre-bound launch of one workload (buffers allocated once, outside the timed region)."""

    def __init__(self, inp, dev, mixed=None):
        """mixed: (num_prefill_seqs, prefill_total_q, prefill_total_k,
        decode_max_seqlen_k) to call mea_fwd_mixed instead of mea_fwd."""
        import torch
        from memory_efficient_attention_amd import _native
        self.inp, self.mixed = inp, mixed
        self.q, self.k, self.v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
        self.ssq, self.ssk = inp.seqstart_q.to(dev), inp.seqstart_k.to(dev)
        self.slopes = None if inp.alibi_slopes is None else inp.alibi_slopes.to(dev)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((inp.Hq, inp.total_q), dtype=torch.float32, device=dev)
        if mixed is None:
            self.ws_bytes = _native.mea_fwd_workspace_size(len(inp.seqlens_q), inp.total_k, inp.max_seqlen_q,
                                                           inp.max_seqlen_k, inp.Hq, inp.Hkv, inp.D, 0)
        else:
            self.ws_bytes = _native.mea_fwd_mixed_workspace_size(len(inp.seqlens_q), inp.total_k, inp.max_seqlen_q,
                                                                 inp.max_seqlen_k, mixed[0], mixed[2], mixed[3],
                                                                 inp.Hq, inp.Hkv, inp.D)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=dev)
        self.dtype = _native.MEA_BF16 if inp.dtype == "bf16" else _native.MEA_F16
        self.native = _native

    def __call__(self, stream):
        inp = self.inp
        head = (self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.out.data_ptr(),
                self.lse.data_ptr(), self.ssq.data_ptr(), self.ssk.data_ptr(), len(inp.seqlens_q),
                inp.total_q, inp.total_k, inp.max_seqlen_q, inp.max_seqlen_k)
        tail = (inp.Hq, inp.Hkv, inp.D, self.dtype, int(inp.causal),
                None if self.slopes is None else self.slopes.data_ptr(), inp.scale,
                self.ws.data_ptr() if self.ws_bytes else None, self.ws_bytes, stream.cuda_stream)
        if self.mixed is None:
            st = self.native.mea_fwd(*head, *tail)
        else:
            st = self.native.mea_fwd_mixed(*head, *self.mixed, *tail)
        if st != 0:
            raise RuntimeError(f"mea_fwd: {self.native.mea_status_string(st)}: {self.native.mea_last_error()}")


PAGE_SIZE = 64   # keys per page of the paged decode variant


class PagedCall:
    """Pre-bound launch of one workload with K/V scattered into a paged cache
    (pages in a seeded random order; see mea_workloads.to_paged)."""

    def __init__(self, inp, dev, page_size):
        import torch
        from memory_efficient_attention_amd import _native
        from mea_workloads import to_paged
        pk = to_paged(inp, page_size, seed=1)
        self.inp, self.page_size = inp, page_size
        self.q = inp.q.to(dev)
        self.kc, self.vc, self.bt = pk.k_cache.to(dev), pk.v_cache.to(dev), pk.block_table.to(dev)
        self.ssq, self.ssk = inp.seqstart_q.to(dev), inp.seqstart_k.to(dev)
        self.slopes = None if inp.alibi_slopes is None else inp.alibi_slopes.to(dev)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((inp.Hq, inp.total_q), dtype=torch.float32, device=dev)
        self.ws_bytes = _native.mea_fwd_workspace_size(len(inp.seqlens_q), inp.total_k, inp.max_seqlen_q,
                                                       inp.max_seqlen_k, inp.Hq, inp.Hkv, inp.D, 0)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=dev)
        self.dtype = _native.MEA_BF16 if inp.dtype == "bf16" else _native.MEA_F16
        self.native = _native

    def __call__(self, stream):
        inp = self.inp
        st = self.native.mea_fwd_paged(
            self.q.data_ptr(), self.kc.data_ptr(), self.vc.data_ptr(), self.out.data_ptr(),
            self.lse.data_ptr(), self.ssq.data_ptr(), self.ssk.data_ptr(), self.bt.data_ptr(),
            len(inp.seqlens_q), inp.total_q, inp.total_k, inp.max_seqlen_q, inp.max_seqlen_k,
            self.page_size, self.kc.shape[0], self.bt.shape[1], inp.Hq, inp.Hkv, inp.D, self.dtype,
            int(inp.causal), None if self.slopes is None else self.slopes.data_ptr(), inp.scale,
            self.ws.data_ptr() if self.ws_bytes else None, self.ws_bytes, stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"mea_fwd_paged: {self.native.mea_status_string(st)}: {self.native.mea_last_error()}")


class PagedFp8Call:
    """Pre-bound mea_fwd_paged_fp8 launch: q, k, v quantised to e4m3 as for
    Fp8Call, the k/v codes scattered into a paged cache as for PagedCall;
    bf16 output."""

    def __init__(self, inp, dev, page_size):
        import dataclasses
        import torch
        from memory_efficient_attention_amd import _native
        from mea_workloads import to_fp8, to_paged
        f = to_fp8(inp)
        pk = to_paged(dataclasses.replace(inp, k=f.k8, v=f.v8), page_size, seed=1)
        self.inp, self.f, self.page_size = inp, f, page_size
        self.q = f.q8.to(dev)
        self.kc, self.vc, self.bt = pk.k_cache.to(dev), pk.v_cache.to(dev), pk.block_table.to(dev)
        self.ssq, self.ssk = inp.seqstart_q.to(dev), inp.seqstart_k.to(dev)
        self.slopes = None if inp.alibi_slopes is None else inp.alibi_slopes.to(dev)
        self.out = torch.empty((inp.total_q, inp.Hq, inp.D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((inp.Hq, inp.total_q), dtype=torch.float32, device=dev)
        self.ws_bytes = _native.mea_fwd_fp8_workspace_size(len(inp.seqlens_q), inp.total_k, inp.max_seqlen_q,
                                                            inp.max_seqlen_k, inp.Hq, inp.Hkv, inp.D)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=dev)
        self.native = _native

    def __call__(self, stream):
        inp, f = self.inp, self.f
        st = self.native.mea_fwd_paged_fp8(
            self.q.data_ptr(), self.kc.data_ptr(), self.vc.data_ptr(), f.q_scale, f.k_scale, f.v_scale,
            self.out.data_ptr(), self.lse.data_ptr(), self.ssq.data_ptr(), self.ssk.data_ptr(), self.bt.data_ptr(),
            len(inp.seqlens_q), inp.total_q, inp.total_k, inp.max_seqlen_q, inp.max_seqlen_k, self.page_size,
            self.kc.shape[0], self.bt.shape[1], inp.Hq, inp.Hkv, inp.D, self.native.MEA_BF16, int(inp.causal),
            None if self.slopes is None else self.slopes.data_ptr(), inp.scale,
            self.ws.data_ptr() if self.ws_bytes else None, self.ws_bytes, stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"mea_fwd_paged_fp8: {self.native.mea_status_string(st)}: "
                               f"{self.native.mea_last_error()}")


class BwdCall:
    """Pre-bound backward launch (mea_bwd) of one workload: out and lse come
    from one forward call at set-up, dO is seeded N(0, 1)."""

    def __init__(self, fwd_call, dev, seed):
        import torch
        from mea_workloads import random_dout
        inp = fwd_call.inp
        fwd_call(torch.cuda.current_stream(dev))
        self.f = fwd_call
        self.inp = inp
        self.dout = random_dout(seed, inp).to(dev)
        self.dq, self.dk, self.dv = (torch.empty_like(x) for x in (self.f.q, self.f.k, self.f.v))
        self.native = fwd_call.native
        self.ws_bytes = self.native.mea_bwd_workspace_size(len(inp.seqlens_q), inp.total_q, inp.total_k, inp.Hq,
                                                           inp.Hkv, inp.D)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=dev)

    def __call__(self, stream):
        inp, f = self.inp, self.f
        st = self.native.mea_bwd(
            f.q.data_ptr(), f.k.data_ptr(), f.v.data_ptr(), f.out.data_ptr(), f.lse.data_ptr(),
            self.dout.data_ptr(), self.dq.data_ptr(), self.dk.data_ptr(), self.dv.data_ptr(),
            f.ssq.data_ptr(), f.ssk.data_ptr(), len(inp.seqlens_q), inp.total_q, inp.total_k,
            inp.max_seqlen_q, inp.max_seqlen_k, inp.Hq, inp.Hkv, inp.D, f.dtype, int(inp.causal),
            None if f.slopes is None else f.slopes.data_ptr(), inp.scale,
            self.ws.data_ptr() if self.ws_bytes else None, self.ws_bytes, stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"mea_bwd: {self.native.mea_status_string(st)}: {self.native.mea_last_error()}")


class Fp8Call:
    """Pre-bound launch of the fp8 forward (mea_fwd_fp8) on a workload whose
    q, k, v are quantised to OCP e4m3 with per-tensor scales; bf16 output."""

    def __init__(self, inp, dev):
        import torch
        from memory_efficient_attention_amd import _native
        from mea_workloads import to_fp8
        f = to_fp8(inp)
        self.inp, self.f = inp, f
        self.q, self.k, self.v = f.q8.to(dev), f.k8.to(dev), f.v8.to(dev)
        self.ssq, self.ssk = inp.seqstart_q.to(dev), inp.seqstart_k.to(dev)
        self.slopes = None if inp.alibi_slopes is None else inp.alibi_slopes.to(dev)
        self.out = torch.empty((inp.total_q, inp.Hq, inp.D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((inp.Hq, inp.total_q), dtype=torch.float32, device=dev)
        self.ws_bytes = _native.mea_fwd_fp8_workspace_size(len(inp.seqlens_q), inp.total_k, inp.max_seqlen_q,
                                                            inp.max_seqlen_k, inp.Hq, inp.Hkv, inp.D)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=dev)
        self.native = _native

    def __call__(self, stream):
        inp, f = self.inp, self.f
        st = self.native.mea_fwd_fp8(
            self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), f.q_scale, f.k_scale, f.v_scale,
            self.out.data_ptr(), self.lse.data_ptr(), self.ssq.data_ptr(), self.ssk.data_ptr(),
            len(inp.seqlens_q), inp.total_q, inp.total_k, inp.max_seqlen_q, inp.max_seqlen_k, inp.Hq, inp.Hkv,
            inp.D, self.native.MEA_BF16, int(inp.causal), None if self.slopes is None else self.slopes.data_ptr(),
            inp.scale, self.ws.data_ptr() if self.ws_bytes else None, self.ws_bytes, stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"mea_fwd_fp8: {self.native.mea_status_string(st)}: {self.native.mea_last_error()}")


PEAK_MFMA_FP8_TFLOPS = 5033.2    # dense fp8 MFMA: twice the bf16 rate
# fp8 forward: Q K^T on fp8 matrix cores, P V on half precision ones; its
# roofline peak is the rate at which the two halves of the FLOPs could run
# back to back: 1 / (0.5 / fp8 peak + 0.5 / bf16 peak)
PEAK_FP8_FWD_TFLOPS = 1.0 / (0.5 / PEAK_MFMA_FP8_TFLOPS + 0.5 / PEAK_MFMA_BF16_TFLOPS)

class FfnCall:
    """Pre-bound SwiGLU feed-forward launch (mea_swiglu_ffn) on the prefill
    workload's tokens: d_model 4096, d_ff 11008, bf16, seeded weights."""

    def __init__(self, dev, seed):
        import torch
        from memory_efficient_attention_amd import _native
        from mea_workloads import FFN_WORKLOAD, swiglu_case
        w = FFN_WORKLOAD
        f = swiglu_case(seed, w["tokens"], w["d_model"], w["d_ff"], dtype=w["dtype"])
        self.shape = (w["tokens"], w["d_model"], w["d_ff"])
        self.x, self.wg, self.wu, self.wd = (t.to(dev) for t in (f.x, f.w_gate, f.w_up, f.w_down))
        self.hidden = torch.empty((w["tokens"], w["d_ff"]), dtype=self.x.dtype, device=dev)
        self.out = torch.empty_like(self.x)
        self.native = _native

    def flops(self) -> int:
        T, d, F = self.shape
        return 6 * T * d * F   # gate, up (2 T d F each) and down (2 T F d)

    def __call__(self, stream):
        T, d, F = self.shape
        st = self.native.mea_swiglu_ffn(self.x.data_ptr(), self.wg.data_ptr(), self.wu.data_ptr(), self.wd.data_ptr(),
                                        self.hidden.data_ptr(), self.out.data_ptr(), T, d, F, self.native.MEA_BF16,
                                        stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"mea_swiglu_ffn: {self.native.mea_status_string(st)}: {self.native.mea_last_error()}")


def mixed_setup(seed, dev):
    """The mixed serving workload (8 prefills U[128, 4096], then 56 decode
    steps over U[1024, 32768] keys, 32/8 heads, D 128, bf16, causal): the
    mea_fwd_mixed call, its prefill part and its decode part each called on
    its own (the same tensors, as sub-batches), and mea_fwd on the whole batch
    (every sequence through the prefill kernels)."""
    from memory_efficient_attention_amd import BlockDiagonalCausalMask
    from mea_workloads import mixed_case, prefix
    inp = mixed_case(seed)
    split = BlockDiagonalCausalMask.from_seqlens(inp.seqlens_q, inp.seqlens_k).mixed_split()
    n_pre = split[0]
    pre = prefix(inp, n_pre)
    dec = suffix(inp, n_pre)
    return {"inp": inp, "pre": pre, "dec": dec, "split": split, "mixed": Call(inp, dev, mixed=split),
            "whole": Call(inp, dev), "pre_call": Call(pre, dev), "dec_call": Call(dec, dev)}


def suffix(inp, n):
    """Sequences n .. end of ``inp`` as their own batch (views of the same tensors)."""
    import dataclasses
    from mea_workloads import seqstart_from_lengths
    sq, sk = inp.seqstart_q.tolist(), inp.seqstart_k.tolist()
    return dataclasses.replace(inp, q=inp.q[sq[n]:], k=inp.k[sk[n]:], v=inp.v[sk[n]:],
                               seqstart_q=seqstart_from_lengths(inp.seqlens_q[n:]),
                               seqstart_k=seqstart_from_lengths(inp.seqlens_k[n:]),
                               seqlens_q=inp.seqlens_q[n:], seqlens_k=inp.seqlens_k[n:], bmghk=None)


def mixed_timings(c, stream, reps):
    pre_flops = unmasked_flops(c["pre"])
    dec_bytes = algorithmic_bytes(c["dec"])
    ms = time_calls(c["mixed"], stream, reps)
    whole_ms = time_calls(c["whole"], stream, reps)
    pms = time_calls(c["pre_call"], stream, reps)
    dms = time_calls(c["dec_call"], stream, reps)
    ptf = pre_flops / (pms * 1e-3) / 1e12
    dgb = dec_bytes / (dms * 1e-3) / 1e9
    inp = c["inp"]
    return {"ms": round(ms, 4), "ms_all_through_prefill_kernels": round(whole_ms, 4),
            "speedup": round(whole_ms / ms, 3),
            "config": {"prefills": c["split"][0], "prefill_tokens": c["split"][1],
                       "decodes": len(inp.seqlens_q) - c["split"][0], "decode_kv_tokens": c["dec"].total_k,
                       "Hq": inp.Hq, "Hkv": inp.Hkv, "D": inp.D, "dtype": inp.dtype, "mask": "block-diagonal causal"},
            "prefill_part": {"ms": round(pms, 4), "value": round(ptf, 2), "unit": "TFLOP/s",
                             "frac": round(ptf / PEAK_MFMA_BF16_TFLOPS, 4), "unmasked_flops": pre_flops},
            "decode_part": {"ms": round(dms, 4), "value": round(dgb, 1), "unit": "GB/s",
                            "frac": round(dgb / PEAK_HBM_GBS, 4), "algorithmic_bytes": dec_bytes},
            "parts_ms_sum": round(pms + dms, 4)}


BWD_GEMMS = 2.5   # backward algorithmic FLOPs / forward's: Q K^T, dO V^T, P^T dO, dS K, dS^T Q vs Q K^T, P V


def time_calls(call, stream, reps):
    """Average ms of `reps` back-to-back calls, HIP events on the launch stream."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    call(stream)
    e0.record(stream)
    for _ in range(reps):
        call(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def host_cpu():
    """CPU model and core counts of this host (Linux /proc and the process's affinity)."""
    model, cores = None, set()
    phys, core = None, None
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                k, _, v = ln.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model is None:
                    model = v
                elif k == "physical id":
                    phys = v
                elif k == "core id":
                    core = v
                elif not k and phys is not None:
                    cores.add((phys, core))
                    phys = core = None
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = None
    return {"cpu_model": model, "physical_cores": len(cores) or None, "logical_cpus": os.cpu_count(),
            "cpus_allowed": allowed}


def _time_oracle(inp):
    import oracle
    t0 = time.perf_counter()
    out, lse = oracle.attention_forward(inp.q, inp.k, inp.v, inp.seqstart_q, inp.seqstart_k, causal=inp.causal,
                                        alibi_slopes=inp.alibi_slopes, scale=inp.scale)
    return time.perf_counter() - t0, out, lse


def cpu_baseline(pre_inp, gpu_out, gpu_lse, budget_s: float, dec_inp=None, dec_budget_s: float = 4.0,
                 small=None, cfg3=None):
    """Time the float64 CPU oracle on the prefill workload's sequences, one at
    a time in order, until about budget_s seconds have been spent (the budget
    plus at most one sequence), and check the GPU rows of those sequences.
    Also: the decode workload's requests the same way (dec_inp, dec_budget_s),
    each small parity workload whole (small: name -> Inputs) and the 4 x 2048
    prefill whole (cfg3), and the host's CPU model and core count.  The
    oracle runs on torch's CPU threads: the host share this process was given
    (OMP_NUM_THREADS), which ``cores`` reports."""
    import torch
    import oracle
    sq, sk = pre_inp.seqstart_q.tolist(), pre_inp.seqstart_k.tolist()
    n_done, flops, dt, err, lerr = 0, 0, 0.0, 0.0, 0.0
    for b in range(len(pre_inp.seqlens_q)):
        if dt >= budget_s:
            break
        Lq, Lk = sq[b + 1] - sq[b], sk[b + 1] - sk[b]
        t0 = time.perf_counter()
        ref_out, ref_lse = oracle.attention_forward(
            pre_inp.q[sq[b]:sq[b + 1]], pre_inp.k[sk[b]:sk[b + 1]], pre_inp.v[sk[b]:sk[b + 1]],
            [0, Lq], [0, Lk], causal=True, scale=pre_inp.scale)
        dt += time.perf_counter() - t0
        flops += 4 * pre_inp.D * pre_inp.Hq * Lq * (Lq + 1) // 2
        err = max(err, (gpu_out[sq[b]:sq[b + 1]].double() - ref_out).abs().max().item())
        lerr = max(lerr, (gpu_lse[:, sq[b]:sq[b + 1]].double() - ref_lse).abs().max().item())
        n_done += 1
    res = {
        "value": flops / dt / 1e12, "unit": "TFLOP/s",
        "cores": torch.get_num_threads(), "kind": "oracle",
        "sample": f"first {n_done} of {len(pre_inp.seqlens_q)} sequences of the prefill workload "
                  f"({sq[n_done]} tokens, {flops / 1e9:.1f} unmasked GFLOP), float64, {dt:.1f} s",
        "gpu_vs_oracle_on_sample": {"max_abs_out": err, "max_abs_lse": lerr},
        "host": host_cpu(),
    }
    if dec_inp is not None:
        n, dbytes, ddt = 0, 0, 0.0
        while n < len(dec_inp.seqlens_q) and ddt < dec_budget_s:
            one = one_sequence(dec_inp, n)
            t, _, _ = _time_oracle(one)
            ddt += t
            dbytes += algorithmic_bytes(one)
            n += 1
        res["decode"] = {"value": dbytes / ddt / 1e9, "unit": "GB/s",
                         "sample": f"first {n} of {len(dec_inp.seqlens_q)} requests of the decode workload "
                                   f"({dec_inp.seqstart_k.tolist()[n]} keys), float64, {ddt:.1f} s"}
    per_config = {}
    for name, inp in (small or {}).items():
        t, _, _ = _time_oracle(inp)
        per_config[name] = {"seconds": round(t, 4), "tflops": unmasked_flops(inp) / t / 1e12}
    if cfg3 is not None:
        t, _, _ = _time_oracle(cfg3)
        per_config[PREFILL_4X2048] = {"seconds": round(t, 3), "tflops": unmasked_flops(cfg3) / t / 1e12}
    if per_config:
        res["per_config"] = per_config
    return res


def one_sequence(inp, b):
    """Sequence b of ``inp`` on its own (views of the same tensors)."""
    import dataclasses
    from mea_workloads import seqstart_from_lengths
    sq, sk = inp.seqstart_q.tolist(), inp.seqstart_k.tolist()
    lq, lk = sq[b + 1] - sq[b], sk[b + 1] - sk[b]
    return dataclasses.replace(inp, q=inp.q[sq[b]:sq[b + 1]], k=inp.k[sk[b]:sk[b + 1]], v=inp.v[sk[b]:sk[b + 1]],
                               seqstart_q=seqstart_from_lengths([lq]), seqstart_k=seqstart_from_lengths([lk]),
                               seqlens_q=[lq], seqlens_k=[lk], bmghk=None)


COPY_BYTES = 1 << 30   # calibration copy: 1 GiB read + 1 GiB written per launch

# Parts whose counter runs make up each reported traffic figure: the kernels of
# one call (warm-up included, averaged per dispatch) and the parts that ran them.
TRAFFIC_PARTS = {
    # (the last two template arguments of fwd_prefill_kernel: the bfloat16-V
    # second launch, and persistent workgroups)
    "fwd_prefill": ("prefill", ["vt_images_kernel<128, true, false, false>",
                                "fwd_prefill_kernel<128, true, true, false, false, false, false, true>",
                                "fwd_prefill_kernel<128, true, true, false, false, false, true, false>"]),
    "fwd_prefill_alibi": ("prefill_alibi", ["vt_images_kernel<128, true, false, false>",
                                            "fwd_prefill_kernel<128, true, true, true, false, false, false, true>",
                                            "fwd_prefill_kernel<128, true, true, true, false, false, true, false>"]),
    "fwd_prefill_4x2048": ("prefill_4x2048", ["vt_images_kernel<128, true, false, false>",
                                              "fwd_prefill_kernel<128, true, true, true, false, false, false, false>",
                                              "fwd_prefill_kernel<128, true, true, true, false, false, true, false>"]),
    "fwd_decode": ("decode", ["fwd_decode_partial_kernel<128, true, false, false, false>",
                              "fwd_decode_combine_kernel<128, true>"]),
    "bwd": ("backward", ["bwd_prep_kernel<128, true>", "bwd_dkdv_kernel<128, true, true, false>",
                         "bwd_dq_kernel<128, true, true, false>"]),
    "fwd_prefill_fp8": ("prefill_fp8", ["vt_images_kernel<128, true, false, true>",
                                        "fwd_prefill_kernel<128, true, true, false, false, true, false, true>"]),
    "fwd_decode_fp8": ("decode_fp8", ["fwd_decode_partial_kernel<128, true, false, false, true>",
                                      "fwd_decode_combine_kernel<128, true>"]),
    "ffn": ("ffn", ["ffn_gemm_kernel<true, true>", "ffn_gemm_kernel<true, false>"]),
}


def _counter_means(path, counter):
    """Mean counter value (KiB) per dispatch of each kernel in one rocprofv3
    --pmc CSV (counter_collection), keyed by the kernel name without the
    namespace and argument list."""
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {path}")
    sums, counts = {}, {}
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                name = row["Kernel_Name"]
                name = name[name.find("::") + 2:] if name.startswith("void mea::") or name.startswith("mea::") else name
                name = name.split("(")[0].strip()
                sums[name] = sums.get(name, 0.0) + float(row["Counter_Value"])
                counts[name] = counts.get(name, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}, counts


TRACE_SUMMARY_FILE = os.path.join(ROOT, "profiles", "bench_default_kernel_stats.md")


def _trace_label(name, segment):
    """Workload of one dispatch of the default run, from its kernel and the
    run's segment: 0 = before the backward, 1 = backward, 2 = the mixed batch,
    3 = fp8, 4 = SwiGLU.  Pre-passes, bfloat16-V second launches and combines
    take the label of their call's main kernel (None here)."""
    if name.startswith(("vt_images_kernel", "fwd_decode_combine_kernel")) or \
            (name.startswith("fwd_prefill_kernel") and name.endswith("true, false>")):
        return None
    if name.startswith("bwd_"):
        return "backward"
    if name.startswith("ffn_gemm_kernel"):
        return "SwiGLU feed-forward"
    if name.startswith("fwd_prefill_kernel"):
        args = [x.strip() for x in name[name.index("<") + 1:-1].split(",")]
        alibi, fp8, persist = args[3] == "true", args[5] == "true", args[7] == "true"
        if fp8:
            return "fp8 prefill"
        if segment == 2:
            return "mixed batch, all through the prefill kernels" if persist else "mixed batch: prefill part"
        if alibi:
            return "prefill + ALiBi" if persist else "4 x 2048 prefill + ALiBi"
        return "prefill (64 sequences)"
    if name.startswith("fwd_decode_partial_kernel"):
        args = [x.strip() for x in name[name.index("<") + 1:-1].split(",")]
        paged, fp8 = args[3] == "true", args[4] == "true"
        if segment == 2:
            return "mixed batch: decode part"
        return ("fp8 " if fp8 else "") + ("decode, 64-key pages" if paged else "decode")
    return "other"


def trace_summary(root, bench_json=None):
    """profiles/bench_default_kernel_stats.md from the kernel trace of one
    rocprofv3 --kernel-trace run of the default bench (and its JSON line)."""
    import csv
    import glob
    import statistics
    files = glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no kernel_trace.csv under {root}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    disp = []
    segment = 0
    for r in rows:
        name = r["Kernel_Name"]
        name = name[name.find("::") + 2:] if "mea::" in name else name
        name = name.split("(")[0].strip()
        if not name.startswith(("fwd_", "bwd_", "vt_images", "ffn_")):
            continue
        if name.startswith("bwd_"):
            segment = 1
        elif segment == 1:
            segment = 2
        if name.startswith("vt_images_kernel") and name.endswith("true>"):
            segment = 3
        if name.startswith("ffn_"):
            segment = 4
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        disp.append([name, _trace_label(name, segment), us])
    # pre-passes take the label of the next main kernel, the rest of the previous
    for i, d in enumerate(disp):
        if d[1] is None and d[0].startswith("vt_images_kernel"):
            d[1] = next((e[1] for e in disp[i + 1:] if e[1] is not None), "other")
    last = "other"
    for d in disp:
        if d[1] is None:
            d[1] = last
        last = d[1]
    groups = {}
    for name, label, us in disp:
        groups.setdefault((label, name), []).append(us)
    lines = ["# Kernel-trace statistics of the default bench run (MI355X, gfx950, one GPU)", "",
             "Command (repository root, `TMPDIR=/tmp`), then the summary:", "",
             "    rocprofv3 --kernel-trace --stats -d DIR -o kt --output-format csv -- python3 bench.py > DIR.json",
             "    python3 bench.py --trace-summary DIR --trace-json DIR.json", "",
             "(DIR: any output directory.)", "",
             "Every dispatch of the run, grouped by the workload it served (the bench's fixed call order:",
             "the step's prefill and decode, the ALiBi prefill, the 4 x 2048 prefill, paged decode,",
             "backward, the mixed batch, fp8, SwiGLU). Warm-up calls are included; \"steady\" leaves",
             "out each group's first two calls. `__amd_rocclr_copyBuffer` (input upload, CPU",
             "baseline copies) is outside every timed region and not listed.", "",
             "| workload | kernel | calls | mean µs | median µs | steady mean µs |",
             "|---|---|---:|---:|---:|---:|"]
    order = []
    for name, label, _ in disp:
        if (label, name) not in order:
            order.append((label, name))
    steady = {}
    for label, name in order:
        v = groups[(label, name)]
        st = v[2:] if len(v) > 4 else v
        steady[(label, name)] = statistics.mean(st)
        lines.append(f"| {label} | `{name}` | {len(v)} | {statistics.mean(v):.1f} | {statistics.median(v):.1f} | "
                     f"{steady[(label, name)]:.1f} |")
    if bench_json is not None:
        with open(bench_json) as fh:
            rec = json.loads(fh.read().strip().splitlines()[-1])
        per_call = {}
        for (label, name), us in steady.items():
            per_call[label] = per_call.get(label, 0.0) + us
        pairs = [("prefill (64 sequences)", rec["roofline"].get("launch_ms")),
                 ("decode", rec.get("decode", {}).get("ms")),
                 ("prefill + ALiBi", (rec.get("prefill_alibi") or {}).get("ms")),
                 ("4 x 2048 prefill + ALiBi", (rec.get("prefill_4x2048") or {}).get("ms")),
                 ("decode, 64-key pages", (rec.get("decode_paged") or {}).get("ms")),
                 ("backward", (rec.get("backward") or {}).get("ms")),
                 ("mixed batch: prefill part", ((rec.get("mixed") or {}).get("prefill_part") or {}).get("ms")),
                 ("mixed batch: decode part", ((rec.get("mixed") or {}).get("decode_part") or {}).get("ms")),
                 ("fp8 prefill", (rec.get("prefill_fp8") or {}).get("ms")),
                 ("fp8 decode", (rec.get("decode_fp8") or {}).get("ms")),
                 ("fp8 decode, 64-key pages", (rec.get("decode_paged_fp8") or {}).get("ms")),
                 ("SwiGLU feed-forward", (rec.get("swiglu_ffn") or {}).get("ms"))]
        lines += ["", "Per call: the steady means of a call's kernels summed, against the bench line's HIP-event",
                  "time of the same call in the same (profiled) run:", "",
                  "| call | kernels, steady (µs) | bench line (µs) |", "|---|---:|---:|"]
        for label, ms in pairs:
            if label in per_call and ms is not None:
                lines.append(f"| {label} | {per_call[label]:.1f} | {ms * 1e3:.1f} |")
        lines += ["", f"The bench line of this run: prefill {rec['value']} {rec['unit']} "
                      f"(frac {rec['roofline']['frac']}), {rec['ms_per_step']} ms per step."]
    with open(TRACE_SUMMARY_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(TRACE_SUMMARY_FILE)


def write_traffic(root):
    """profiles/hbm_traffic.json from the FETCH_SIZE / WRITE_SIZE runs under
    root: each counter scaled by what it reads for the copy of known size."""
    fetch_copy, _ = _counter_means(os.path.join(root, "pmc_copy_FETCH_SIZE"), "FETCH_SIZE")
    write_copy, _ = _counter_means(os.path.join(root, "pmc_copy_WRITE_SIZE"), "WRITE_SIZE")
    fk = max(fetch_copy.values())
    wk = max(write_copy.values())
    fetch_factor = COPY_BYTES / (fk * 1024)
    write_factor = COPY_BYTES / (wk * 1024)
    rec = {"source_hash": kernel_source_hash(),
           "calibration": {"copy_bytes_each_way": COPY_BYTES, "fetch_kib_per_dispatch": fk,
                           "write_kib_per_dispatch": wk, "fetch_factor": round(fetch_factor, 4),
                           "write_factor": round(write_factor, 4)},
           "per_kernel": {}, "kernels": {}}
    for key, (part, kernels) in TRAFFIC_PARTS.items():
        try:
            fetch, nf = _counter_means(os.path.join(root, f"pmc_{part}_FETCH_SIZE"), "FETCH_SIZE")
            write, _ = _counter_means(os.path.join(root, f"pmc_{part}_WRITE_SIZE"), "WRITE_SIZE")
        except FileNotFoundError:
            continue
        per, total = {}, 0
        for k in kernels:
            if k not in fetch:
                continue
            rb = int(fetch[k] * 1024 * fetch_factor)
            wb = int(write.get(k, 0.0) * 1024 * write_factor)
            per[k] = {"read_bytes": rb, "write_bytes": wb, "dispatches": nf[k]}
            total += rb + wb
        rec["per_kernel"][key] = per
        rec["kernels"][key] = total
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec["kernels"]))


def run_part(args, dev):
    """Time one half of the step on its own (profiling aid); prints a short JSON line.

    ``--part copy`` runs a plain device-to-device copy of COPY_BYTES instead: the
    known-size kernel that scales the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    from mea_workloads import generate
    if args.part == "copy":
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        stream = torch.cuda.current_stream(dev)
        for _ in range(args.warmup):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / max(args.steps, 1)
        print(json.dumps({"part": "copy", "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                          "ms": round(ms, 4), "gbs": round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 1)}),
              flush=True)
        return
    name = PREFILL if args.part in ("prefill", "backward", "prefill_fp8") else DECODE
    if args.part == "prefill_alibi":
        call = Call(generate(PREFILL, seed=args.seed, alibi=True), dev)
    elif args.part == "prefill_4x2048":
        call = Call(generate(PREFILL_4X2048, seed=args.seed), dev)
    elif args.part == "ffn":
        call = FfnCall(dev, args.seed)
    elif args.part in ("prefill_fp8", "decode_fp8"):
        call = Fp8Call(generate(name, seed=args.seed), dev)
    elif args.part == "decode_paged":
        call = PagedCall(generate(name, seed=args.seed), dev, PAGE_SIZE)
    elif args.part == "decode_paged_fp8":
        call = PagedFp8Call(generate(name, seed=args.seed), dev, PAGE_SIZE)
    elif args.part == "backward":
        call = BwdCall(Call(generate(name, seed=args.seed), dev), dev, args.seed)
    else:
        call = Call(generate(name, seed=args.seed), dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        call(stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        call(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / max(args.steps, 1)
    workload = {"ffn": "swiglu_ffn", "prefill_4x2048": PREFILL_4X2048, "prefill_alibi": PREFILL + " + alibi"}
    res = {"part": args.part, "workload": workload.get(args.part, name), "ms": round(ms, 4)}
    if args.part in ("decode_paged", "decode_paged_fp8"):
        res["page_size"] = PAGE_SIZE
    if args.part in ("prefill", "prefill_fp8", "prefill_alibi", "prefill_4x2048"):
        res["tflops"] = round(unmasked_flops(call.inp) / (ms * 1e-3) / 1e12, 2)
    elif args.part == "backward":
        res["tflops"] = round(BWD_GEMMS * unmasked_flops(call.inp) / (ms * 1e-3) / 1e12, 2)
    elif args.part == "ffn":
        res["tflops"] = round(call.flops() / (ms * 1e-3) / 1e12, 2)
    elif args.part in ("decode_fp8", "decode_paged_fp8"):
        res["gbs"] = round(algorithmic_bytes_fp8(call.inp) / (ms * 1e-3) / 1e9, 1)
    else:
        res["gbs"] = round(algorithmic_bytes(call.inp) / (ms * 1e-3) / 1e9, 1)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of CPU oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-alibi-variant", action="store_true")
    ap.add_argument("--no-paged-variant", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-ffn", action="store_true")
    ap.add_argument("--no-mixed", action="store_true")
    ap.add_argument("--write-traffic", metavar="DIR", default=None,
                    help="write profiles/hbm_traffic.json from the rocprofv3 counter runs under DIR and exit "
                         "(no GPU needed)")
    ap.add_argument("--trace-summary", metavar="DIR", default=None,
                    help="write profiles/bench_default_kernel_stats.md from the rocprofv3 kernel trace of a "
                         "default run under DIR and exit (no GPU needed)")
    ap.add_argument("--trace-json", metavar="FILE", default=None,
                    help="with --trace-summary: the JSON line that profiled run printed")
    ap.add_argument("--part", choices=["all", "prefill", "decode", "decode_paged", "backward", "prefill_fp8",
                                       "decode_fp8", "decode_paged_fp8", "ffn", "prefill_alibi", "prefill_4x2048",
                                       "copy"],
                    default="all",
                    help="run only one half of the step, or the calibration copy (for profiling); "
                         "the JSON line is for 'all'")
    args = ap.parse_args()
    if args.write_traffic is not None:
        write_traffic(args.write_traffic)
        return
    if args.trace_summary is not None:
        trace_summary(args.trace_summary, args.trace_json)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: there is no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)

    import torch
    from mea_workloads import generate
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.part != "all":
        run_part(args, dev)
        return

    t_gen = time.perf_counter()
    pre = generate(PREFILL, seed=args.seed)
    dec = generate(DECODE, seed=args.seed)
    pre_call, dec_call = Call(pre, dev), Call(dec, dev)
    pre_alibi = None
    if not args.no_alibi_variant:
        pre_alibi = Call(generate(PREFILL, seed=args.seed, alibi=True), dev)
    dec_paged = None
    if not args.no_paged_variant:
        dec_paged = PagedCall(dec, dev, PAGE_SIZE)
    bwd_call = None
    if not args.no_backward:
        bwd_call = BwdCall(Call(pre, dev), dev, args.seed)
    fp8_call = fp8_dec_call = fp8_paged_call = None
    if not args.no_fp8:
        fp8_call = Fp8Call(pre, dev)
        fp8_dec_call = Fp8Call(dec, dev)
        if not args.no_paged_variant:
            fp8_paged_call = PagedFp8Call(dec, dev, PAGE_SIZE)
    ffn_call = None
    if not args.no_ffn:
        ffn_call = FfnCall(dev, args.seed)
    cfg3 = generate(PREFILL_4X2048, seed=args.seed)
    cfg3_call = Call(cfg3, dev)
    mixed_calls = None
    if not args.no_mixed:
        mixed_calls = mixed_setup(args.seed, dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs generated and resident in HBM in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        pre_call(stream)
        dec_call(stream)
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        pre_call(stream)
        ev[i][1].record(stream)
        dec_call(stream)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    print(f"[bench] {K} steps: prefill {pre_ms:.3f} ms, decode {dec_ms:.3f} ms per step",
          file=sys.stderr, flush=True)

    pre_flops = unmasked_flops(pre)
    dec_bytes = algorithmic_bytes(dec)
    tflops = pre_flops / (pre_ms * 1e-3) / 1e12
    gbs = dec_bytes / (dec_ms * 1e-3) / 1e9

    alibi_res = None
    if pre_alibi is not None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        pre_alibi(stream)
        e0.record(stream)
        for _ in range(max(3, K // 3)):
            pre_alibi(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ams = e0.elapsed_time(e1) / max(3, K // 3)
        atf = unmasked_flops(pre_alibi.inp) / (ams * 1e-3) / 1e12
        alibi_res = {"ms": round(ams, 4), "tflops": round(atf, 2),
                     "frac": round(atf / PEAK_MFMA_BF16_TFLOPS, 4),
                     "roofline": {"bound": "mfma", "achieved": round(atf, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(atf / PEAK_MFMA_BF16_TFLOPS, 4),
                                  "traffic": measured_traffic("fwd_prefill_alibi"),
                                  "kernel": "mea_fwd prefill call with ALiBi: vt_images_kernel + "
                                            "fwd_prefill_kernel<128,bf16,causal,alibi>"}}

    # the 4 x 2048 causal ALiBi GQA prefill: short sequences, so the grid is
    # four rounds of workgroups and its fixed costs weigh more
    c3ms = time_calls(cfg3_call, stream, max(20, 2 * K))
    c3tf = unmasked_flops(cfg3) / (c3ms * 1e-3) / 1e12
    cfg3_res = {"ms": round(c3ms, 4), "value": round(c3tf, 2), "unit": "TFLOP/s",
                "config": {"seqs": 4, "tokens": cfg3.total_q, "Hq": 32, "Hkv": 8, "D": 128, "dtype": "bf16",
                           "mask": "block-diagonal causal", "alibi": True, "unmasked_flops": unmasked_flops(cfg3)},
                "roofline": {"bound": "mfma", "achieved": round(c3tf, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(c3tf / PEAK_MFMA_BF16_TFLOPS, 4),
                             "traffic": measured_traffic("fwd_prefill_4x2048"),
                             "kernel": "mea_fwd prefill call with ALiBi: vt_images_kernel + "
                                       "fwd_prefill_kernel<128,bf16,causal,alibi>"}}

    paged_res = None
    if dec_paged is not None:  # the decode workload with K/V in shuffled pages of PAGE_SIZE keys
        pms = time_calls(dec_paged, stream, max(5, K // 2))
        pgb = dec_bytes / (pms * 1e-3) / 1e9
        paged_res = {"page_size": PAGE_SIZE, "ms": round(pms, 4), "value": round(pgb, 1), "unit": "GB/s",
                     "frac": round(pgb / PEAK_HBM_GBS, 4)}

    bwd_res = None
    if bwd_call is not None:  # the prefill workload's gradients (dq, dk, dv) from a seeded dO
        bms = time_calls(bwd_call, stream, max(3, K // 3))
        btf = BWD_GEMMS * pre_flops / (bms * 1e-3) / 1e12
        bwd_res = {"ms": round(bms, 4), "value": round(btf, 2), "unit": "TFLOP/s",
                   "roofline": {"bound": "mfma", "achieved": round(btf, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
                                "unit": "TFLOP/s", "frac": round(btf / PEAK_MFMA_BF16_TFLOPS, 4),
                                "traffic": measured_traffic("bwd"),
                                "kernel": "mea_bwd call: bwd_prep_kernel + bwd_dkdv_kernel + bwd_dq_kernel "
                                          "<128,bf16,causal>"},
                   "algorithmic_flops": int(BWD_GEMMS * pre_flops)}

    mixed_res = None
    if mixed_calls is not None:
        mixed_res = mixed_timings(mixed_calls, stream, max(5, K // 2))

    fp8_res = None
    if fp8_call is not None:  # the prefill workload with q, k, v in e4m3 and per-tensor scales
        fms = time_calls(fp8_call, stream, max(5, K // 2))
        ftf = pre_flops / (fms * 1e-3) / 1e12
        fp8_res = {"ms": round(fms, 4), "value": round(ftf, 2), "unit": "TFLOP/s",
                   "roofline": {"bound": "mfma", "achieved": round(ftf, 2), "peak": round(PEAK_FP8_FWD_TFLOPS, 1),
                                "unit": "TFLOP/s", "frac": round(ftf / PEAK_FP8_FWD_TFLOPS, 4),
                                "traffic": measured_traffic("fwd_prefill_fp8"),
                                "kernel": "mea_fwd_fp8 call: vt_images_kernel<fp8> + fwd_prefill_kernel<128,bf16 out,"
                                          "causal,fp8>"}}

    fp8_dec_res = None
    if fp8_dec_call is not None:  # the decode workload with q, k, v in e4m3: half the K/V bytes
        dfms = time_calls(fp8_dec_call, stream, max(5, K // 2))
        dfb = algorithmic_bytes_fp8(dec)
        dfgb = dfb / (dfms * 1e-3) / 1e9
        fp8_dec_res = {"ms": round(dfms, 4), "value": round(dfgb, 1), "unit": "GB/s",
                       "speedup_vs_bf16_decode": round(dec_ms / dfms, 3), "algorithmic_bytes": dfb,
                       "roofline": {"bound": "hbm", "achieved": round(dfgb, 1), "peak": PEAK_HBM_GBS,
                                    "unit": "GB/s", "frac": round(dfgb / PEAK_HBM_GBS, 4),
                                    "traffic": measured_traffic("fwd_decode_fp8"),
                                    "kernel": "mea_fwd_fp8 decode call: fwd_decode_partial_kernel<128,bf16 out,"
                                              "fp8> + fwd_decode_combine_kernel"}}

    fp8_paged_res = None
    if fp8_paged_call is not None:  # the same in shuffled pages of PAGE_SIZE keys
        pfms = time_calls(fp8_paged_call, stream, max(5, K // 2))
        pfgb = algorithmic_bytes_fp8(dec) / (pfms * 1e-3) / 1e9
        fp8_paged_res = {"page_size": PAGE_SIZE, "ms": round(pfms, 4), "value": round(pfgb, 1), "unit": "GB/s",
                         "frac": round(pfgb / PEAK_HBM_GBS, 4)}

    ffn_res = None
    if ffn_call is not None:  # the SwiGLU feed-forward layer on the prefill workload's tokens
        nms = time_calls(ffn_call, stream, max(3, K // 6))
        ntf = ffn_call.flops() / (nms * 1e-3) / 1e12
        T, d, F = ffn_call.shape
        ffn_res = {"ms": round(nms, 4), "value": round(ntf, 2), "unit": "TFLOP/s",
                   "config": {"tokens": T, "d_model": d, "d_ff": F, "dtype": "bf16", "flops": ffn_call.flops()},
                   "roofline": {"bound": "mfma", "achieved": round(ntf, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
                                "unit": "TFLOP/s", "frac": round(ntf / PEAK_MFMA_BF16_TFLOPS, 4),
                                "traffic": measured_traffic("ffn"),
                                "kernel": "mea_swiglu_ffn call: ffn_gemm_kernel<bf16,gated> + ffn_gemm_kernel<bf16>"}}

    traffic_pre = measured_traffic("fwd_prefill")
    traffic_dec = measured_traffic("fwd_decode")
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{PREFILL} + {DECODE}",
            "prefill": {"seqs": 64, "tokens": pre.total_q, "Hq": 32, "Hkv": 8, "D": 128,
                        "mask": "block-diagonal causal", "alibi": False,
                        "unmasked_flops": pre_flops},
            "decode": {"requests": 64, "kv_tokens": dec.total_k, "Hq": 64, "Hkv": 8, "D": 128,
                       "algorithmic_bytes": dec_bytes,
                       "chunk_keys": dec_call.native.mea_default_chunk_keys(dec.total_k, 64, 8)},
            "seed": args.seed,
        },
        "roofline": {
            "bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_BF16_TFLOPS, 4),
            "traffic": traffic_pre,
            "kernel": "mea_fwd prefill call: vt_images_kernel + fwd_prefill_kernel<128,bf16,causal>",
            "launch_ms": round(pre_ms, 4),
        },
        "decode": {
            "value": round(gbs, 1), "unit": "GB/s", "ms": round(dec_ms, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": traffic_dec,
                         "kernel": "fwd_decode_partial_kernel + fwd_decode_combine_kernel"},
        },
        "prefill_alibi": alibi_res,
        "prefill_4x2048": cfg3_res,
        "mixed": mixed_res,
        "backward": bwd_res,
        "prefill_fp8": fp8_res,
        "decode_fp8": fp8_dec_res,
        "swiglu_ffn": ffn_res,
        "decode_paged": paged_res,
        "decode_paged_fp8": fp8_paged_res,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(pre, pre_call.out.cpu(), pre_call.lse.cpu(), args.cpu_budget,
                                            dec_inp=dec, small={n: generate(n, seed=args.seed) for n in SMALL_WORKLOADS},
                                            cfg3=cfg3)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
