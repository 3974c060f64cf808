"""Pins for the SwiGLU feed-forward oracle (``oracle.ffn``).

  * brute force: scalar loops with math.fsum and math.exp on tiny inputs;
  * a library routine: torch.nn.functional.silu and linear in float64;
  * closed forms: SiLU(0) = 0, SiLU(z) -> z for large z and -> 0 for very
    negative z, SiLU(1) = 1 / (1 + 1/e); a zero gate or a zero up projection
    gives a zero output; with w_gate scaled so the gate is large, the layer
    reduces to the bilinear (x Wg^T) * (x Wu^T) W_down^T;
  * mutation tests: planted mistakes in a copy of the oracle must each fail.
"""
import math
import os
import types

import pytest
import torch

import oracle
from oracle.ffn import silu, swiglu_ffn
from mea_workloads import swiglu_case

FFN_SRC = os.path.join(os.path.dirname(oracle.__file__), "ffn.py")


def brute(x, wg, wu, wd):
    X, G, U, Dn = (t.double().tolist() for t in (x, wg, wu, wd))
    T, dm, df = len(X), len(X[0]), len(G)
    hid = [[0.0] * df for _ in range(T)]
    out = [[0.0] * dm for _ in range(T)]
    for t in range(T):
        for f in range(df):
            g = math.fsum(X[t][i] * G[f][i] for i in range(dm))
            u = math.fsum(X[t][i] * U[f][i] for i in range(dm))
            hid[t][f] = g / (1.0 + math.exp(-g)) * u
        for j in range(dm):
            out[t][j] = math.fsum(hid[t][f] * Dn[j][f] for f in range(df))
    return torch.tensor(hid, dtype=torch.float64), torch.tensor(out, dtype=torch.float64)


CASES = [(3, 4, 6), (5, 8, 3), (1, 16, 16), (7, 5, 9)]


def _brute_ok(fn, ci):
    T, dm, df = CASES[ci]
    f = swiglu_case(100 + ci, T, dm, df, dtype="bf16")
    h, o, _ = fn(f.x, f.w_gate, f.w_up, f.w_down)
    bh, bo = brute(f.x, f.w_gate, f.w_up, f.w_down)
    return (h - bh).abs().max().item() < 1e-12 and (o - bo).abs().max().item() < 1e-12


def _library_ok(fn, seed=5):
    F = torch.nn.functional
    f = swiglu_case(seed, 33, 64, 96, dtype="fp16")
    h, o, _ = fn(f.x, f.w_gate, f.w_up, f.w_down)
    X, Wg, Wu, Wd = (t.double() for t in (f.x, f.w_gate, f.w_up, f.w_down))
    ref_h = F.silu(F.linear(X, Wg)) * F.linear(X, Wu)
    ref_o = F.linear(ref_h, Wd)
    return (h - ref_h).abs().max().item() < 1e-12 and (o - ref_o).abs().max().item() < 1e-12


def _special_ok(fn):
    f = swiglu_case(9, 6, 8, 10, dtype="bf16")
    zero = torch.zeros_like(f.w_gate)
    _, o1, _ = fn(f.x, zero, f.w_up, f.w_down)      # SiLU(0) = 0
    _, o2, _ = fn(f.x, f.w_gate, zero, f.w_down)    # up = 0
    # large positive gate: SiLU(z) = z (to 1e-30 relative); make the gate x Wg^T >= 100 by a ramp input
    x = torch.ones((2, 8), dtype=torch.float64)
    wg = torch.full((10, 8), 20.0, dtype=torch.float64)
    wu = f.w_up.double()
    wd = f.w_down.double()
    h3, o3, _ = fn(x, wg, wu, wd)
    g = x @ wg.T
    ok3 = (h3 - g * (x @ wu.T)).abs().max().item() < 1e-9
    return o1.abs().max().item() == 0 and o2.abs().max().item() == 0 and ok3


def test_silu_closed_forms():
    z = torch.tensor([0.0, 1.0, -1.0, 50.0, -800.0], dtype=torch.float64)
    s = silu(z)
    assert s[0].item() == 0.0
    assert abs(s[1].item() - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(s[2].item() - (-1.0 / (1.0 + math.e))) < 1e-15
    assert abs(s[3].item() - 50.0) < 1e-15
    assert s[4].item() == 0.0 or abs(s[4].item()) < 1e-300


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_brute_force(ci):
    assert _brute_ok(swiglu_ffn, ci)


def test_library_routine():
    assert _library_ok(swiglu_ffn)


def test_special_cases():
    assert _special_ok(swiglu_ffn)


def test_out_abs_bounds_out():
    f = swiglu_case(3, 9, 16, 24)
    _, o, a = swiglu_ffn(f.x, f.w_gate, f.w_up, f.w_down)
    assert bool((o.abs() <= a + 1e-12).all())


MUTATIONS = [
    ("return z / (1.0 + torch.exp(-z))", "return 1.0 / (1.0 + torch.exp(-z))"),   # sigmoid for SiLU
    ("return z / (1.0 + torch.exp(-z))", "return z / (1.0 + torch.exp(z))"),       # sign in the exponent
    ("hidden = silu(gate) * up", "hidden = silu(up) * gate"),                      # gate and up swapped
    ("hidden = silu(gate) * up", "hidden = gate * up"),                            # gate not activated
    ("out = hidden @ Wd.transpose(0, 1)", "out = hidden @ Wd.transpose(0, 1) + hidden.sum() * 0 + 1e-9"),
    ("gate = X @ Wg.transpose(0, 1)", "gate = X @ Wu.transpose(0, 1)"),            # wrong weight
]


def _mutant(old, new):
    src = open(FFN_SRC).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("ffn_mutant")
    mod.__dict__["math"] = math
    exec(compile(src.replace(old, new), "ffn_mutant", "exec"), mod.__dict__)
    return mod.swiglu_ffn


def _pins_pass(fn):
    try:
        return all(_brute_ok(fn, ci) for ci in range(len(CASES))) and _library_ok(fn) and _special_ok(fn)
    except Exception:
        return False


def test_unmutated_ffn_oracle_passes_pins():
    assert _pins_pass(swiglu_ffn)


@pytest.mark.parametrize("mi", range(len(MUTATIONS)))
def test_planted_ffn_mistake_fails_pins(mi):
    assert not _pins_pass(_mutant(*MUTATIONS[mi]))


# ---- out_abs and the row-sampled form (the full-size GPU check uses both) ----

def brute_out_abs(x, wg, wu, wd):
    """sum_f |hidden[t, f] * w_down[j, f]| by scalar loops and math.fsum."""
    h, _ = brute(x, wg, wu, wd)
    H, Dn = h.tolist(), wd.double().tolist()
    T, df, dm = len(H), len(H[0]), len(Dn)
    return torch.tensor([[math.fsum(abs(H[t][f] * Dn[j][f]) for f in range(df)) for j in range(dm)]
                         for t in range(T)], dtype=torch.float64)


def _out_abs_ok(fn):
    for ci in range(len(CASES)):
        T, dm, df = CASES[ci]
        f = swiglu_case(200 + ci, T, dm, df, dtype="bf16")
        _, _, a = fn(f.x, f.w_gate, f.w_up, f.w_down)
        ba = brute_out_abs(f.x, f.w_gate, f.w_up, f.w_down)
        # equal in both directions, relative to each element's own size
        if not bool(((a - ba).abs() <= 1e-12 * ba.abs().clamp_min(1e-300)).all()):
            return False
    return True


ROWS = [6, 0, 6, 12, 3, 0]   # unsorted, repeated, the first (0) and the last (12) token


def _rows_ok(fn_rows):
    f = swiglu_case(300, 13, 8, 10, dtype="bf16")
    idx = torch.tensor(ROWS)
    h, o, a = fn_rows(f.x, f.w_gate, f.w_up, f.w_down, ROWS)
    bh, bo = brute(f.x[idx], f.w_gate, f.w_up, f.w_down)
    ba = brute_out_abs(f.x[idx], f.w_gate, f.w_up, f.w_down)
    if h.shape != (len(ROWS), 10) or o.shape != (len(ROWS), 8) or a.shape != (len(ROWS), 8):
        return False
    return ((h - bh).abs().max().item() < 1e-12 and (o - bo).abs().max().item() < 1e-12
            and (a - ba).abs().max().item() < 1e-12)


def test_out_abs_brute_force():
    assert _out_abs_ok(swiglu_ffn)


def test_rows_brute_force():
    assert _rows_ok(oracle.swiglu_ffn_rows)


def test_rows_equal_full_rows():
    """The row-sampled form returns the full layer's rows (same float64 arithmetic)."""
    f = swiglu_case(301, 40, 16, 24, dtype="bf16")
    rows = [39, 0, 17, 17, 5]
    full = swiglu_ffn(f.x, f.w_gate, f.w_up, f.w_down)
    part = oracle.swiglu_ffn_rows(f.x, f.w_gate, f.w_up, f.w_down, rows)
    for a, b in zip(part, full):
        assert (a - b[torch.tensor(rows)]).abs().max().item() < 1e-12


ROW_MUTATIONS = [
    # the error scale of each output element inflated: it loosens every GPU bound built on it
    ("out_abs = hidden.abs() @ Wd.abs().transpose(0, 1)", "out_abs = 100 * (hidden.abs() @ Wd.abs().transpose(0, 1))"),
    # the scale without absolute values inside the sum
    ("out_abs = hidden.abs() @ Wd.abs().transpose(0, 1)", "out_abs = (hidden @ Wd.transpose(0, 1)).abs()"),
    # the first len(rows) tokens instead of the selected ones
    ("return swiglu_ffn(x[idx], w_gate, w_up, w_down)", "return swiglu_ffn(x[:len(idx)], w_gate, w_up, w_down)"),
]


def _mutant_module(old, new):
    src = open(FFN_SRC).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("ffn_mutant")
    exec(compile(src.replace(old, new), "ffn_mutant", "exec"), mod.__dict__)
    return mod


def _row_pins_pass(mod):
    try:
        return _out_abs_ok(mod.swiglu_ffn) and _rows_ok(mod.swiglu_ffn_rows)
    except Exception:
        return False


def test_unmutated_row_pins_pass():
    assert _row_pins_pass(oracle.ffn)


@pytest.mark.parametrize("mi", range(len(ROW_MUTATIONS)))
def test_planted_row_mistake_fails_pins(mi):
    assert not _row_pins_pass(_mutant_module(*ROW_MUTATIONS[mi]))
