"""GPU parity of the SwiGLU feed-forward layer (``mea_swiglu_ffn``) against
the float64 oracle, element by element on small shapes with ragged token
counts, and on sampled token rows at the full size.

Bounds, with u the unit roundoff of the dtype (2^-8 for bf16, 2^-11 for
fp16: the largest relative error of one rounding to nearest):
  hidden:  |h - h_ref| <= 2u |h_ref| + 1e-3 u max|h_ref|
           (one rounding of hidden, plus as much again for the float32
           accumulation of gate and up and the float32 SiLU)
  out:     |o - o_ref| <= 2u sum_f |h_f w_jf| + 2u |o_ref| + 1e-3 u max|o_ref|
           (each hidden term enters the second product rounded; out is
           rounded once; the same allowance again)"""
import sys

import pytest
import torch

import oracle
from mea_workloads import FFN_WORKLOAD, swiglu_case

pytestmark = pytest.mark.gpu

U = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _run(f):
    from memory_efficient_attention_amd import swiglu_ffn
    dev = "cuda"
    T, dm = f.x.shape
    dff = f.w_gate.shape[0]
    hidden = torch.full((T, dff), float("nan"), dtype=f.x.dtype, device=dev)
    out = torch.full((T, dm), float("nan"), dtype=f.x.dtype, device=dev)
    swiglu_ffn(f.x.to(dev), f.w_gate.to(dev), f.w_up.to(dev), f.w_down.to(dev), hidden=hidden, out=out)
    torch.cuda.synchronize()
    return hidden.cpu().double(), out.cpu().double()


def _check(h, o, rh, ro, ra, dtype, what):
    u = U[dtype]
    assert not torch.isnan(h).any() and not torch.isnan(o).any(), f"{what}: unwritten elements"
    eh = (h - rh).abs()
    bh = 2 * u * rh.abs() + 1e-3 * u * rh.abs().max()
    eo = (o - ro).abs()
    bo = 2 * u * ra + 2 * u * ro.abs() + 1e-3 * u * ro.abs().max()
    worst_h = (eh / bh).max().item()
    worst_o = (eo / bo).max().item()
    res = {"max_abs_hidden": eh.max().item(), "max_abs_out": eo.max().item(),
           "hidden_err_over_bound": worst_h, "out_err_over_bound": worst_o}
    assert worst_h <= 1.0, f"{what}: hidden error {eh.max().item():.3e} exceeds its bound ({res})"
    assert worst_o <= 1.0, f"{what}: out error {eo.max().item():.3e} exceeds its bound ({res})"
    return res


CASES = [
    # (tokens, d_model, d_ff, dtype)
    (1, 256, 128, "bf16"),
    (255, 256, 384, "bf16"),
    (300, 512, 640, "fp16"),
    (1000, 256, 256, "bf16"),
    (513, 768, 1152, "bf16"),
    (2048, 1024, 2816, "bf16"),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_ffn_parity(ci):
    T, dm, dff, dt = CASES[ci]
    f = swiglu_case(900 + ci, T, dm, dff, dtype=dt)
    _log(f"ffn T={T} d_model={dm} d_ff={dff} {dt}")
    h, o = _run(f)
    rh, ro, ra = oracle.swiglu_ffn(f.x, f.w_gate, f.w_up, f.w_down)
    _log(f"  {_check(h, o, rh, ro, ra, dt, f'ffn case {ci}')}")


def test_ffn_deterministic():
    f = swiglu_case(950, 300, 256, 384)
    a, b = _run(f), _run(f)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_ffn_full_size_sampled():
    """137,663 tokens x d_model 4096 x d_ff 11008 (bf16); 64 sampled rows, the
    first and last token included."""
    w = FFN_WORKLOAD
    f = swiglu_case(0, w["tokens"], w["d_model"], w["d_ff"], dtype=w["dtype"])
    _log("ffn full size")
    h, o = _run(f)
    g = torch.Generator().manual_seed(4)
    rows = sorted(set([0, w["tokens"] - 1] + torch.randint(0, w["tokens"], (62,), generator=g).tolist()))
    rh, ro, ra = oracle.swiglu_ffn_rows(f.x, f.w_gate, f.w_up, f.w_down, rows)
    idx = torch.tensor(rows)
    _log(f"  {_check(h[idx], o[idx], rh, ro, ra, 'bf16', 'ffn full size')}")
