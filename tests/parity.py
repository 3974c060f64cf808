"""Helpers shared by the GPU parity tests: run the HIP path through the
Python binding and compare it element by element with the CPU oracle."""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import torch

import oracle
from mea_workloads import Inputs

# Tolerances on N(0,1) inputs: max-abs error of out vs the float64 oracle,
# and of the finite log-sum-exps; rows with no key must have lse == -inf exactly.
OUT_TOL = {"fp16": 2e-3, "bf16": 1e-2}
LSE_TOL = 1e-3


def to_device(inp: Inputs, device="cuda"):
    return dict(
        q=inp.q.to(device), k=inp.k.to(device), v=inp.v.to(device),
        seqstart_q=inp.seqstart_q.to(device), seqstart_k=inp.seqstart_k.to(device),
        slopes=None if inp.alibi_slopes is None else inp.alibi_slopes.to(device))


def run_gpu(inp: Inputs, dev: Optional[dict] = None, chunk_keys: Optional[int] = None,
            poison: bool = True, return_lse: bool = True):
    """One call through ``attention_packed``; out is pre-filled with NaN so
    that any row the kernels fail to write shows up."""
    from memory_efficient_attention_amd import attention_packed
    d = dev or to_device(inp)
    out = torch.full_like(d["q"], float("nan")) if poison else None
    res = attention_packed(d["q"], d["k"], d["v"], d["seqstart_q"], d["seqstart_k"],
                           inp.max_seqlen_q, inp.max_seqlen_k, causal=inp.causal,
                           alibi_slopes=d["slopes"], scale=inp.scale, return_lse=return_lse,
                           out=out, chunk_keys=chunk_keys)
    torch.cuda.synchronize()
    if return_lse:
        return res[0].cpu(), res[1].cpu()
    return res.cpu(), None


def oracle_full(inp: Inputs):
    return oracle.attention_forward(inp.q, inp.k, inp.v, inp.seqstart_q, inp.seqstart_k,
                                    causal=inp.causal, alibi_slopes=inp.alibi_slopes,
                                    scale=inp.scale)


def compare(out_gpu: torch.Tensor, lse_gpu: Optional[torch.Tensor], ref_out: torch.Tensor,
            ref_lse: torch.Tensor, dtype: str, what: str = "") -> dict:
    """Assert parity; returns the error figures for reporting."""
    assert out_gpu.shape == ref_out.shape, (what, out_gpu.shape, ref_out.shape)
    o = out_gpu.double()
    assert not torch.isnan(o).any(), f"{what}: NaN in out (unwritten or invalid rows)"
    err = (o - ref_out).abs()
    max_err = err.max().item() if err.numel() else 0.0
    n_bad = int((err > OUT_TOL[dtype]).sum())
    res = {"max_abs_out": max_err, "n_over_tol": n_bad}
    if lse_gpu is not None:
        l = lse_gpu.double()
        ref_inf = torch.isneginf(ref_lse)
        assert torch.equal(torch.isneginf(l), ref_inf), f"{what}: -inf lse rows differ"
        fin = ~ref_inf
        lerr = (l[fin] - ref_lse[fin]).abs().max().item() if fin.any() else 0.0
        assert not torch.isnan(l).any(), f"{what}: NaN in lse"
        res["max_abs_lse"] = lerr
        assert lerr <= LSE_TOL, f"{what}: lse error {lerr:.3e} > {LSE_TOL}"
    assert max_err <= OUT_TOL[dtype], f"{what}: out error {max_err:.3e} > {OUT_TOL[dtype]} ({n_bad} elements)"
    return res


def compare_rows(out_gpu: torch.Tensor, lse_gpu: torch.Tensor, inp: Inputs,
                 rows: Sequence[Tuple[int, int]], what: str = "") -> dict:
    """Sampled parity: the oracle evaluates only the given (token, head) rows."""
    ro, rl = oracle.attention_rows(inp.q, inp.k, inp.v, inp.seqstart_q, inp.seqstart_k, rows,
                                   causal=inp.causal, alibi_slopes=inp.alibi_slopes,
                                   scale=inp.scale)
    go = torch.stack([out_gpu[t, h] for t, h in rows])
    gl = torch.stack([lse_gpu[h, t] for t, h in rows])
    return compare(go, gl, ro, rl, inp.dtype, what)


# Backward tolerance.  Q K^T and dO V^T run in the input precision with
# float32 accumulation; P and dS are rounded to the input precision (unit
# roundoff u: 2^-11 for fp16, 2^-8 for bf16) before the second products,
# rowsum(dO * out) is formed from the rounded forward output, and dq, dk, dv
# are rounded once more on output.  Two bounds must both hold:
#   per tensor:  |g - g_ref| <= 4u max|g_ref| + 1e-6
#   per element: |g - g_ref| <= 4u A + 2u |g_ref| + 1e-6
# where A is the oracle's error scale of that element (the sum of the sizes
# of its terms, P and |dS| taken no smaller than the type's smallest normal
# number, below which a rounding errs by up to u times that number).  The
# element-wise bound catches a row left wrong or zero whose values sit far
# below the tensor's largest.
GRAD_TOL_REL = {"fp16": 4 * 2.0 ** -11, "bf16": 4 * 2.0 ** -8}
UNIT_ROUNDOFF = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}
SMALLEST_NORMAL = {"fp16": 2.0 ** -14, "bf16": 2.0 ** -126}


def run_gpu_backward(inp: Inputs, dout: torch.Tensor, dev: Optional[dict] = None):
    """Forward (out, lse) then backward through the HIP library; dq, dk, dv
    are pre-filled with NaN so that any row the kernels fail to write shows up."""
    from memory_efficient_attention_amd import attention_backward_packed, attention_packed
    d = dev or to_device(inp)
    out, lse = attention_packed(d["q"], d["k"], d["v"], d["seqstart_q"], d["seqstart_k"],
                                inp.max_seqlen_q, inp.max_seqlen_k, causal=inp.causal,
                                alibi_slopes=d["slopes"], scale=inp.scale, return_lse=True)
    nan = float("nan")
    dq = torch.full_like(d["q"], nan)
    dk = torch.full_like(d["k"], nan)
    dv = torch.full_like(d["v"], nan)
    attention_backward_packed(d["q"], d["k"], d["v"], out, lse, dout.to(d["q"].device), d["seqstart_q"],
                              d["seqstart_k"], inp.max_seqlen_q, inp.max_seqlen_k, causal=inp.causal,
                              alibi_slopes=d["slopes"], scale=inp.scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


class GradRef(tuple):
    """The oracle's (dq, dk, dv), with their element-wise error scales in
    ``.scales``."""
    scales = None


def oracle_backward(inp: Inputs, dout: torch.Tensor) -> GradRef:
    kw = dict(causal=inp.causal, alibi_slopes=inp.alibi_slopes, scale=inp.scale)
    args = (inp.q, inp.k, inp.v, dout, inp.seqstart_q, inp.seqstart_k)
    ref = GradRef(oracle.attention_backward(*args, **kw))
    ref.scales = oracle.attention_backward_scales(*args, **kw, floor=SMALLEST_NORMAL[inp.dtype])
    return ref


def compare_grads(got, ref, dtype: str, what: str = "") -> dict:
    """Assert parity of (dq, dk, dv) with the oracle's; returns error figures
    (max error, max |ref|, and the worst error over its element-wise bound)."""
    res = {}
    u = UNIT_ROUNDOFF[dtype]
    scales = getattr(ref, "scales", None)
    assert scales is not None, f"{what}: the oracle reference carries no error scales"
    for name, g, r, a in zip(("dq", "dk", "dv"), got, ref, scales):
        assert g.shape == r.shape, (what, name, g.shape, r.shape)
        gd = g.double()
        assert not torch.isnan(gd).any(), f"{what}: NaN in {name} (unwritten or invalid rows)"
        scale = r.abs().max().item() if r.numel() else 0.0
        tol = GRAD_TOL_REL[dtype] * scale + 1e-6
        e = (gd - r).abs()
        err = e.max().item() if r.numel() else 0.0
        elem_bound = 4 * u * a + 2 * u * r.abs() + 1e-6
        worst = (e / elem_bound).max().item() if r.numel() else 0.0
        res[name] = (err, scale, round(worst, 3))
        assert err <= tol, f"{what}: {name} error {err:.3e} > {tol:.3e} (max |ref| {scale:.3e})"
        assert worst <= 1.0, (f"{what}: {name} exceeds its element-wise bound by {worst:.2f}x "
                              f"(max error {err:.3e})")
    return res
