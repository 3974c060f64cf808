"""Pins for the oracle's backward (``attention_backward``) against facts that
do not come from the oracle's own gradient formulas.

  * finite differences: central differences of sum(out * dout) through the
    pinned forward, entry by entry, on tiny inputs that include empty
    sequences, rows with no allowed key, GQA, ALiBi and L_q != L_k;
  * a library routine: float64 autograd through torch's
    scaled_dot_product_attention with an additive ALiBi + causal bias and
    enable_gqa (the call the GQA page checks against repeat_interleave);
  * invariants: a softmax is unchanged by adding a constant to every score of
    a row, so the key gradients of a sequence sum to zero; every live softmax
    row sums to one, so the value gradients of a sequence sum to the dO rows
    of the live query rows of the group's heads;
  * mutation tests: plausible mistakes planted in a copy of the oracle's
    backward must each fail one of the pins above.
"""
import math
import os
import types

import pytest
import torch

import oracle
from oracle import attention_backward, attention_forward
from mea_workloads import random_case, random_dout

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "attention.py")

CASES = [
    # (seqlens_q, seqlens_k, Hq, Hkv, D, causal, alibi)
    ([5, 1, 7], None, 4, 2, 8, False, False),
    ([5, 1, 7], None, 4, 2, 8, True, False),
    ([6, 0, 3, 9], None, 4, 1, 8, True, True),        # MQA, empty sequence
    ([4, 8], None, 3, 3, 8, False, True),             # MHA, non-causal ALiBi
    ([1, 1, 1], [9, 4, 12], 4, 2, 8, True, True),     # decode rows (L_q=1 < L_k)
    ([3, 5], [7, 2], 2, 1, 8, True, False),           # L_q > L_k: rows with no key
    ([2, 6], [5, 6], 4, 2, 4, True, True),            # L_q < L_k prefill
    ([2, 0], [0, 3], 2, 2, 4, False, False),          # empty K for a non-empty Q
]


def _case(ci, seed):
    lq, lk, Hq, Hkv, D, causal, alibi = CASES[ci]
    slopes = None
    if alibi:
        slopes = torch.tensor([0.3 + 0.17 * h for h in range(Hq)], dtype=torch.float32)
    inp = random_case(seed, lq, lk, Hq=Hq, Hkv=Hkv, D=D, dtype="fp16", causal=causal,
                      alibi=alibi, slopes=slopes, scale=0.37)
    return inp, random_dout(seed, inp)


def _bwd(fn, inp, dout):
    return fn(inp.q, inp.k, inp.v, dout, inp.seqstart_q, inp.seqstart_k, causal=inp.causal,
              alibi_slopes=inp.alibi_slopes, scale=inp.scale)


def _loss(inp, dout64, q, k, v):
    out, _ = attention_forward(q, k, v, inp.seqstart_q, inp.seqstart_k, causal=inp.causal,
                               alibi_slopes=inp.alibi_slopes, scale=inp.scale)
    return math.fsum((out * dout64).flatten().tolist())


def _finite_differences(inp, dout, eps=1e-6):
    """Central differences of sum(out * dout) for every entry of q, k and v."""
    base = [inp.q.double(), inp.k.double(), inp.v.double()]
    d64 = dout.double()
    grads = []
    for which in range(3):
        g = torch.zeros_like(base[which])
        flat = g.view(-1)
        for i in range(flat.numel()):
            args_p = [t.clone() for t in base]
            args_m = [t.clone() for t in base]
            args_p[which].view(-1)[i] += eps
            args_m[which].view(-1)[i] -= eps
            flat[i] = (_loss(inp, d64, *args_p) - _loss(inp, d64, *args_m)) / (2 * eps)
        grads.append(g)
    return grads


def _fd_ok(fn, ci, seed):
    inp, dout = _case(ci, seed)
    mine = _bwd(fn, inp, dout)
    ref = _finite_differences(inp, dout)
    return all((m - r).abs().max().item() < 1e-6 for m, r in zip(mine, ref))


def _sdpa_autograd(inp, dout):
    """float64 gradients of sum(out * dout) through torch's SDPA, per sequence;
    None for a case with a row that has no allowed key (SDPA gives NaN there)."""
    F = torch.nn.functional
    sq, sk = inp.seqstart_q.tolist(), inp.seqstart_k.tolist()
    dq = torch.zeros(inp.q.shape, dtype=torch.float64)
    dk = torch.zeros(inp.k.shape, dtype=torch.float64)
    dv = torch.zeros(inp.v.shape, dtype=torch.float64)
    for b in range(len(sq) - 1):
        Lq, Lk = sq[b + 1] - sq[b], sk[b + 1] - sk[b]
        if Lq == 0:
            continue
        if Lk == 0:
            return None
        Q = inp.q[sq[b]:sq[b + 1]].double().permute(1, 0, 2)[None].requires_grad_()
        K = inp.k[sk[b]:sk[b + 1]].double().permute(1, 0, 2)[None].requires_grad_()
        V = inp.v[sk[b]:sk[b + 1]].double().permute(1, 0, 2)[None].requires_grad_()
        i = torch.arange(Lq, dtype=torch.float64)[:, None] + (Lk - Lq)
        j = torch.arange(Lk, dtype=torch.float64)[None, :]
        bias = torch.zeros(inp.Hq, Lq, Lk, dtype=torch.float64)
        if inp.alibi_slopes is not None:
            bias = bias - inp.alibi_slopes.double()[:, None, None] * (i - j).abs()[None]
        if inp.causal:
            bias = bias.masked_fill((j > i)[None], float("-inf"))
        if torch.isneginf(bias).all(dim=-1).any():
            return None
        out = F.scaled_dot_product_attention(Q, K, V, attn_mask=bias[None], scale=inp.scale,
                                             enable_gqa=True)
        dO = dout[sq[b]:sq[b + 1]].double().permute(1, 0, 2)[None]
        out.backward(dO)
        dq[sq[b]:sq[b + 1]] = Q.grad[0].permute(1, 0, 2)
        dk[sk[b]:sk[b + 1]] = K.grad[0].permute(1, 0, 2)
        dv[sk[b]:sk[b + 1]] = V.grad[0].permute(1, 0, 2)
    return dq, dk, dv


def _sdpa_ok(fn, ci, seed):
    inp, dout = _case(ci, seed)
    ref = _sdpa_autograd(inp, dout)
    if ref is None:
        return True
    mine = _bwd(fn, inp, dout)
    return all((m - r).abs().max().item() < 1e-12 for m, r in zip(mine, ref))


def _invariants_ok(fn, ci, seed):
    inp, dout = _case(ci, seed)
    dq, dk, dv = _bwd(fn, inp, dout)
    _, lse = attention_forward(inp.q, inp.k, inp.v, inp.seqstart_q, inp.seqstart_k,
                               causal=inp.causal, alibi_slopes=inp.alibi_slopes, scale=inp.scale)
    live = ~torch.isneginf(lse)                                  # [Hq, Tq]
    per_group = inp.Hq // inp.Hkv
    sq, sk = inp.seqstart_q.tolist(), inp.seqstart_k.tolist()
    ok = True
    for b in range(len(sq) - 1):
        for g in range(inp.Hkv):
            ok &= dk[sk[b]:sk[b + 1], g].sum(dim=0).abs().max().item() < 1e-12 if sk[b + 1] > sk[b] else True
            want = torch.zeros(inp.D, dtype=torch.float64)
            for h in range(g * per_group, (g + 1) * per_group):
                rows = live[h, sq[b]:sq[b + 1]]
                want += dout[sq[b]:sq[b + 1], h].double()[rows].sum(dim=0)
            got = dv[sk[b]:sk[b + 1], g].sum(dim=0)
            ok &= (got - want).abs().max().item() < 1e-12
    # rows with no allowed key have no gradient
    ok &= bool((dq.permute(1, 0, 2)[~live] == 0).all())
    return ok


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_finite_differences(ci):
    assert _fd_ok(attention_backward, ci, seed=ci)


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_sdpa_autograd(ci):
    inp, dout = _case(ci, seed=50 + ci)
    ref = _sdpa_autograd(inp, dout)
    if ref is None:
        pytest.skip("a row has no allowed key: SDPA is undefined there (covered by finite differences)")
    mine = _bwd(attention_backward, inp, dout)
    for m, r in zip(mine, ref):
        assert (m - r).abs().max().item() < 1e-12


def test_sdpa_autograd_medium():
    inp = random_case(11, [64, 130, 1, 77], Hq=8, Hkv=2, D=32, dtype="bf16", causal=True,
                      alibi=True)
    dout = random_dout(11, inp)
    ref = _sdpa_autograd(inp, dout)
    mine = _bwd(attention_backward, inp, dout)
    for m, r in zip(mine, ref):
        assert (m - r).abs().max().item() < 1e-11


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_gradient_invariants(ci):
    assert _invariants_ok(attention_backward, ci, seed=80 + ci)


# ----------------------------------------------------------------------------- mutation tests
MUTATIONS = [
    ("dS = P * (dP - (P * dP).sum(dim=1, keepdim=True))", "dS = P * (dP + (P * dP).sum(dim=1, keepdim=True))"),
    ("dS = P * (dP - (P * dP).sum(dim=1, keepdim=True))", "dS = P * (dP - dP.sum(dim=1, keepdim=True))"),
    ("dS = P * (dP - (P * dP).sum(dim=1, keepdim=True))", "dS = P * dP"),
    ("dq[sq[b]:sq[b + 1], h, :] = scale * (dS @ Kg)", "dq[sq[b]:sq[b + 1], h, :] = dS @ Kg"),
    ("dk[sk[b]:sk[b + 1], g, :] += scale * (dS.transpose(0, 1) @ Qh)",
     "dk[sk[b]:sk[b + 1], g, :] = scale * (dS.transpose(0, 1) @ Qh)"),           # group sum dropped
    ("dv[sk[b]:sk[b + 1], g, :] += P.transpose(0, 1) @ dOh",
     "dv[sk[b]:sk[b + 1], g, :] += P.transpose(0, 1) @ dOh.flip(0)"),            # dO rows misaligned
    ("dP = dOh @ Vg.transpose(0, 1)", "dP = dOh @ Kg.transpose(0, 1)"),          # V and K swapped
    ("Kg = K64[sk[b]:sk[b + 1], g, :]\n            Vg", "Kg = K64[sk[b]:sk[b + 1], 0, :]\n            Vg"),
    ("P, _ = _softmax_block(Qh, Kg, qpos, causal, None if slopes is None else slopes[h],",
     "P, _ = _softmax_block(Qh, Kg, qpos, False, None if slopes is None else slopes[h],"),
    ("P, _ = _softmax_block(Qh, Kg, qpos, causal, None if slopes is None else slopes[h],",
     "P, _ = _softmax_block(Qh, Kg, qpos, causal, None if slopes is None else slopes[0],"),
]


def _mutant(old, new):
    src = open(ORACLE_SRC).read()
    start = src.index("def attention_backward")
    head, body = src[:start], src[start:]
    assert body.count(old) >= 1, old
    mod = types.ModuleType("oracle_bwd_mutant")
    mod.__dict__["math"] = math
    exec(compile(head + body.replace(old, new), "oracle_bwd_mutant", "exec"), mod.__dict__)
    return mod.attention_backward


def _pins_pass(fn):
    try:
        for ci in range(len(CASES)):
            if not (_sdpa_ok(fn, ci, 300 + ci) and _invariants_ok(fn, ci, 300 + ci)):
                return False
        return _fd_ok(fn, 5, 399)
    except Exception:
        return False


def test_unmutated_backward_passes_pins():
    assert _pins_pass(attention_backward)


@pytest.mark.parametrize("mi", range(len(MUTATIONS)))
def test_planted_backward_mistake_fails_pins(mi):
    old, new = MUTATIONS[mi]
    assert not _pins_pass(_mutant(old, new))


# ----------------------------------------------------------------------------- error scales
# ``attention_backward_scales`` sums the absolute values of the terms of each
# gradient element (the element-wise GPU bounds are built on it).  Its pins:
# a scalar brute force that lists every term of every element, checks that the
# terms add up to the (finite-difference-pinned) gradient, and sums their
# absolute values; and |gradient| <= its scale.

def _brute_terms(inp, dout, floor):
    """Per element: (sum of the terms, sum of their sizes), by scalar loops."""
    from oracle import attention_forward
    out, _ = attention_forward(inp.q, inp.k, inp.v, inp.seqstart_q, inp.seqstart_k, causal=inp.causal,
                               alibi_slopes=inp.alibi_slopes, scale=inp.scale)
    Q, K, V, dO, O = (t.double().tolist() for t in (inp.q, inp.k, inp.v, dout, out))
    Hq, Hkv, D, sc = inp.Hq, inp.Hkv, inp.D, inp.scale
    sl = None if inp.alibi_slopes is None else inp.alibi_slopes.double().tolist()
    sq, sk = inp.seqstart_q.tolist(), inp.seqstart_k.tolist()
    tq = {}
    tk = {}
    tv = {}
    for b in range(len(sq) - 1):
        Lq, Lk = sq[b + 1] - sq[b], sk[b + 1] - sk[b]
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for r in range(Lq):
                i = sq[b] + r
                pos = r + Lk - Lq
                keys = [j for j in range(Lk) if not (inp.causal and j > pos)]
                if not keys:
                    continue
                s = {}
                for j in keys:
                    x = sc * math.fsum(Q[i][h][d] * K[sk[b] + j][g][d] for d in range(D))
                    if sl is not None:
                        x -= sl[h] * abs(pos - j)
                    s[j] = x
                m = max(s.values())
                z = math.fsum(math.exp(s[j] - m) for j in keys)
                P = {j: math.exp(s[j] - m) / z for j in keys}
                dP = {j: math.fsum(dO[i][h][d] * V[sk[b] + j][g][d] for d in range(D)) for j in keys}
                rs = math.fsum(P[j] * dP[j] for j in keys)
                dS = {j: P[j] * (dP[j] - rs) for j in keys}
                E = math.fsum(abs(dO[i][h][d] * O[i][h][d]) for d in range(D))
                for j in keys:
                    kj = sk[b] + j
                    p, dd = max(P[j], floor), max(abs(dS[j]), floor)
                    for d in range(D):
                        tq.setdefault((i, h, d), []).append((sc * dS[j] * K[kj][g][d],
                                                             sc * (dd + p * E) * abs(K[kj][g][d])))
                        tk.setdefault((kj, g, d), []).append((sc * dS[j] * Q[i][h][d],
                                                              sc * (dd + p * E) * abs(Q[i][h][d])))
                        tv.setdefault((kj, g, d), []).append((P[j] * dO[i][h][d], p * abs(dO[i][h][d])))
    return tq, tk, tv


def _scales_ok(scales_fn, ci, seed, floor):
    inp, dout = _case(ci, seed)
    args = (inp.q, inp.k, inp.v, dout, inp.seqstart_q, inp.seqstart_k)
    kw = dict(causal=inp.causal, alibi_slopes=inp.alibi_slopes, scale=inp.scale)
    grads = attention_backward(*args, **kw)
    scales = scales_fn(*args, **kw, floor=floor)
    for grad, scl, terms in zip(grads, scales, _brute_terms(inp, dout, floor)):
        want_g = torch.zeros_like(grad)
        want_s = torch.zeros_like(scl)
        for idx, ts in terms.items():
            want_g[idx] = math.fsum(t for t, _ in ts)
            want_s[idx] = math.fsum(a for _, a in ts)
        if (want_g - grad).abs().max().item() > 1e-12:      # the terms are those of the gradient
            return False
        if not bool(((scl - want_s).abs() <= 1e-12 * want_s.abs().clamp_min(1.0)).all()):
            return False
        if floor == 0.0 and not bool((grad.abs() <= scl + 1e-12).all()):
            return False
    return True


SCALE_CASES = [0, 2, 4, 5, 6, 7]   # plain, MQA + empty sequence, decode rows, rows with no key, L_q < L_k, empty K


@pytest.mark.parametrize("ci", SCALE_CASES)
@pytest.mark.parametrize("floor", [0.0, 2.0 ** -6])
def test_backward_scales_brute_force(ci, floor):
    assert _scales_ok(oracle.attention_backward_scales, ci, 700 + ci, floor)


SCALE_MUTATIONS = [
    ("d = torch.where(live, dS.abs().clamp_min(floor), 0.0)", "d = torch.where(live, dS.clamp_min(floor), 0.0)"),
    ("aq[sq[b]:sq[b + 1], h, :] = scale * ((d + p * E) @ Kg.abs())",
     "aq[sq[b]:sq[b + 1], h, :] = scale * (d @ Kg.abs())"),                  # row term dropped
    ("p = torch.where(live, P.clamp_min(floor), 0.0)", "p = P.clamp_min(floor)"),   # floor on masked pairs
    ("av[sk[b]:sk[b + 1], g, :] += p.transpose(0, 1) @ dOh.abs()",
     "av[sk[b]:sk[b + 1], g, :] += 100 * (p.transpose(0, 1) @ dOh.abs())"),  # inflated scale
    ("ak[sk[b]:sk[b + 1], g, :] += scale * ((d + p * E).transpose(0, 1) @ Qh.abs())",
     "ak[sk[b]:sk[b + 1], g, :] = scale * ((d + p * E).transpose(0, 1) @ Qh.abs())"),  # group sum dropped
]


def _scales_mutant(old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_scales_mutant")
    exec(compile(src.replace(old, new), "oracle_scales_mutant", "exec"), mod.__dict__)
    return mod.attention_backward_scales


def _scale_pins_pass(fn):
    try:
        return all(_scales_ok(fn, ci, 800 + ci, fl) for ci in SCALE_CASES for fl in (0.0, 2.0 ** -6))
    except Exception:
        return False


def test_unmutated_scales_pass_pins():
    assert _scale_pins_pass(oracle.attention_backward_scales)


@pytest.mark.parametrize("mi", range(len(SCALE_MUTATIONS)))
def test_planted_scale_mistake_fails_pins(mi):
    assert not _scale_pins_pass(_scales_mutant(*SCALE_MUTATIONS[mi]))
