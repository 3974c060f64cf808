"""Pins for the oracle's fp8 forward (``attention_forward_fp8``).

  * the format: every one of the 256 OCP e4m3 codes decodes (through
    torch.float8_e4m3fn, the routine the oracle relies on) to the value the
    format defines -- sign, 4 exponent bits with bias 7, 3 mantissa bits,
    subnormals at exponent 0, S.1111.111 = NaN, no infinities;
  * scaled inputs: with power-of-two scales every dequantised value is an
    IEEE half, so the fp8 oracle must equal the 16-bit oracle on those halves
    (this fixes which scale multiplies which tensor);
  * homogeneity: doubling v_scale doubles out and leaves lse; swapping q_scale
    and k_scale changes nothing; doubling q_scale equals doubling the score
    scale;
  * mutation tests: planted mistakes in a copy of the fp8 oracle must fail.
"""
import math
import os
import types

import pytest
import torch

import oracle
from oracle import attention_forward, attention_forward_fp8
from mea_workloads import random_case, to_fp8

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "attention.py")


def _ocp_e4m3(code: int) -> float:
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def test_e4m3_decoding_matches_the_format():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    got = codes.to(torch.float64).tolist()
    for c in range(256):
        want = _ocp_e4m3(c)
        assert (math.isnan(want) and math.isnan(got[c])) or got[c] == want, (hex(c), got[c], want)
    assert max(abs(x) for x in got if not math.isnan(x)) == 448.0


CASES = [
    ([5, 1, 7], None, 4, 2, False, False),
    ([6, 0, 3, 9], None, 4, 1, True, True),
    ([1, 1, 1], [9, 4, 12], 4, 2, True, True),
    ([3, 5], [7, 2], 2, 1, True, False),
]


def _case(ci, seed):
    lq, lk, Hq, Hkv, causal, alibi = CASES[ci]
    slopes = torch.tensor([0.3 + 0.17 * h for h in range(Hq)], dtype=torch.float32) if alibi else None
    inp = random_case(seed, lq, lk, Hq=Hq, Hkv=Hkv, D=8, dtype="bf16", causal=causal, alibi=alibi,
                      slopes=slopes, scale=0.37)
    return inp, to_fp8(inp)


def _run8(fn, inp, f, qs, ks, vs, scale=None):
    return fn(f.q8, f.k8, f.v8, qs, ks, vs, inp.seqstart_q, inp.seqstart_k, causal=inp.causal,
              alibi_slopes=inp.alibi_slopes, scale=inp.scale if scale is None else scale)


def _same(a, b, tol=1e-12):
    fa, fb = torch.isfinite(a), torch.isfinite(b)
    return torch.equal(fa, fb) and torch.equal(a[~fa], b[~fb]) and (
        not fa.any() or (a[fa] - b[fb]).abs().max().item() <= tol)


def _pow2_ok(fn, ci):
    inp, f = _case(ci, 10 + ci)
    qs, ks, vs = 0.25, 2.0, 0.125
    halves = [(x.to(torch.float64) * s).to(torch.float16) for x, s in ((f.q8, qs), (f.k8, ks), (f.v8, vs))]
    for x, h, s in zip((f.q8, f.k8, f.v8), halves, (qs, ks, vs)):
        assert torch.equal(h.to(torch.float64), x.to(torch.float64) * s)   # exactly representable
    o8, l8 = _run8(fn, inp, f, qs, ks, vs)
    o16, l16 = attention_forward(*halves, inp.seqstart_q, inp.seqstart_k, causal=inp.causal,
                                 alibi_slopes=inp.alibi_slopes, scale=inp.scale)
    return _same(o8, o16) and _same(l8, l16)


def _homogeneity_ok(fn, ci):
    inp, f = _case(ci, 20 + ci)
    qs, ks, vs = f.q_scale, f.k_scale, f.v_scale
    o, l = _run8(fn, inp, f, qs, ks, vs)
    o2, l2 = _run8(fn, inp, f, qs, ks, 2 * vs)
    o3, l3 = _run8(fn, inp, f, ks, qs, vs)
    o4, l4 = _run8(fn, inp, f, 2 * qs, ks, vs)
    o5, l5 = _run8(fn, inp, f, qs, ks, vs, scale=2 * inp.scale)
    return (_same(o2, 2 * o) and _same(l2, l) and _same(o3, o, 1e-12) and _same(l3, l, 1e-12)
            and _same(o4, o5, 1e-12) and _same(l4, l5, 1e-12))


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_power_of_two_scales_equal_the_16bit_oracle(ci):
    assert _pow2_ok(attention_forward_fp8, ci)


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_scale_homogeneity(ci):
    assert _homogeneity_ok(attention_forward_fp8, ci)


MUTATIONS = [
    ("v = _f64(v8) * float(v_scale)", "v = _f64(v8)"),                          # v_scale dropped
    ("k = _f64(k8) * float(k_scale)", "k = _f64(k8) * float(q_scale)"),         # wrong scale on k
    ("q = _f64(q8) * float(q_scale)", "q = _f64(q8) * float(v_scale)"),         # wrong scale on q
    ("v = _f64(v8) * float(v_scale)", "v = _f64(v8) * float(k_scale)"),         # wrong scale on v
    ("k = _f64(k8) * float(k_scale)", "k = _f64(k8) * float(k_scale) ** 2"),    # scale applied twice
]


def _mutant(old, new):
    src = open(ORACLE_SRC).read()
    start = src.index("def attention_forward_fp8")
    head, body = src[:start], src[start:]
    assert body.count(old) == 1, old
    mod = types.ModuleType("oracle_fp8_mutant")
    mod.__dict__["math"] = math
    exec(compile(head + body.replace(old, new), "oracle_fp8_mutant", "exec"), mod.__dict__)
    return mod.attention_forward_fp8


def _pins_pass(fn):
    try:
        return all(_pow2_ok(fn, ci) and _homogeneity_ok(fn, ci) for ci in range(len(CASES)))
    except Exception:
        return False


def test_unmutated_fp8_oracle_passes_pins():
    assert _pins_pass(attention_forward_fp8)


@pytest.mark.parametrize("mi", range(len(MUTATIONS)))
def test_planted_fp8_mistake_fails_pins(mi):
    assert not _pins_pass(_mutant(*MUTATIONS[mi]))
