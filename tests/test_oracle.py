"""Pins for the CPU oracle against facts that do not come from the oracle itself.

Each check cites the page passage or the mathematics it rests on:
  * brute force: scalar loops with exactly-rounded sums (math.fsum) on tiny
    inputs, including empty and length-1 sequences, GQA, ALiBi, causal and
    L_q != L_k;
  * a library routine: torch's scaled_dot_product_attention in float64 with
    an explicit additive bias and enable_gqa, the same call the GQA page checks
    against repeat_interleave ("group query attention gqa", the enable_gqa
    snippet);
  * closed forms: constant V, identical keys, q = 0 under causal ALiBi
    (a geometric series);
  * invariants: packed == per-sequence (xFormers tutorial section 4), GQA ==
    MHA after repeat_interleave (GQA page), MQA == GQA-1 and MHA == GQA-H
    (GQA-G definition), causality (changing future keys leaves a row
    unchanged), split-KV log-sum-exp combine identity, decode == last row of
    the causal prefill;
  * mutation tests: plausible mistakes planted in a copy of the oracle's source
    must each fail one of the pins above.
"""
import math
import os
import random
import types

import pytest
import torch

import oracle
from oracle import attention_forward, attention_rows
from mea_workloads import random_case, alibi_slopes, seqstart_from_lengths, generate

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "attention.py")


# ----------------------------------------------------------------------------- brute force
def brute_force(q, k, v, seqstart_q, seqstart_k, causal, slopes, scale):
    """Scalar restatement: every score, mask test and exponential written out
    one element at a time, with math.fsum for every sum."""
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    qd, kd, vd = q.double().tolist(), k.double().tolist(), v.double().tolist()
    sl = None if slopes is None else [float(x) for x in slopes.double()]
    sq, sk = seqstart_q.tolist(), seqstart_k.tolist()
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(Tq)]
    lse = [[float("-inf")] * Tq for _ in range(Hq)]
    for b in range(len(sq) - 1):
        Lq, Lk = sq[b + 1] - sq[b], sk[b + 1] - sk[b]
        for r in range(Lq):
            t = sq[b] + r
            i = r + (Lk - Lq)
            for h in range(Hq):
                g = (h * Hkv) // Hq
                scores, keys = [], []
                for j in range(Lk):
                    if causal and j > i:
                        continue
                    s = scale * math.fsum(qd[t][h][d] * kd[sk[b] + j][g][d] for d in range(D))
                    if sl is not None:
                        s -= sl[h] * abs(i - j)
                    scores.append(s)
                    keys.append(sk[b] + j)
                if not scores:
                    continue
                m = max(scores)
                z = math.fsum(math.exp(s - m) for s in scores)
                L = m + math.log(z)
                lse[h][t] = L
                w = [math.exp(s - L) for s in scores]
                for d in range(D):
                    out[t][h][d] = math.fsum(wj * vd[kj][g][d] for wj, kj in zip(w, keys))
    return torch.tensor(out, dtype=torch.float64), torch.tensor(lse, dtype=torch.float64)


def _same(a, b, tol):
    """Equal within tol, with -inf matching -inf exactly."""
    if a.shape != b.shape:
        return False
    fin_a, fin_b = torch.isfinite(a), torch.isfinite(b)
    if not torch.equal(fin_a, fin_b):
        return False
    if not torch.equal(a[~fin_a], b[~fin_b]):
        return False
    if fin_a.any() and (a[fin_a] - b[fin_b]).abs().max().item() > tol:
        return False
    return True


TINY_CASES = [
    # (seqlens_q, seqlens_k, Hq, Hkv, D, causal, alibi)
    ([5, 1, 7], None, 4, 2, 8, False, False),
    ([5, 1, 7], None, 4, 2, 8, True, False),
    ([6, 0, 3, 9], None, 4, 1, 16, True, True),       # MQA, empty sequence
    ([4, 8], None, 3, 3, 8, False, True),             # MHA, non-causal ALiBi
    ([1, 1, 1], [9, 4, 12], 4, 2, 8, True, True),     # decode rows (L_q=1 < L_k)
    ([3, 5], [7, 2], 2, 1, 8, True, False),           # L_q > L_k: rows with no key
    ([16], None, 4, 4, 16, True, True),
    ([2, 0], [0, 3], 2, 2, 4, False, False),          # empty K for a non-empty Q
]


def _tiny(case, seed):
    lq, lk, Hq, Hkv, D, causal, alibi = case
    slopes = None
    if alibi:
        # distinct slopes per head, not the default formula, to catch head mix-ups
        slopes = torch.tensor([0.3 + 0.17 * h for h in range(Hq)], dtype=torch.float32)
    return random_case(seed, lq, lk, Hq=Hq, Hkv=Hkv, D=D, dtype="fp16", causal=causal,
                       alibi=alibi, slopes=slopes, scale=0.37)


def _run(fwd, inp):
    return fwd(inp.q, inp.k, inp.v, inp.seqstart_q, inp.seqstart_k, causal=inp.causal,
               alibi_slopes=inp.alibi_slopes, scale=inp.scale)


@pytest.mark.parametrize("ci", range(len(TINY_CASES)))
def test_brute_force_tiny(ci):
    inp = _tiny(TINY_CASES[ci], seed=ci)
    out, lse = _run(attention_forward, inp)
    bo, bl = brute_force(inp.q, inp.k, inp.v, inp.seqstart_q, inp.seqstart_k, inp.causal,
                         inp.alibi_slopes, inp.scale)
    assert _same(out, bo, 1e-12)
    assert _same(lse, bl, 1e-12)


def test_rows_equal_full():
    inp = random_case(3, [11, 0, 5, 20], [11, 0, 9, 20], Hq=6, Hkv=2, D=16, dtype="bf16",
                      causal=True, alibi=True)
    out, lse = _run(attention_forward, inp)
    rows = [(t, h) for t in range(inp.total_q) for h in range(inp.Hq)]
    ro, rl = attention_rows(inp.q, inp.k, inp.v, inp.seqstart_q, inp.seqstart_k, rows,
                            causal=True, alibi_slopes=inp.alibi_slopes, scale=inp.scale)
    for n, (t, h) in enumerate(rows):
        assert torch.equal(ro[n], out[t, h])
        assert ro[n].shape == out[t, h].shape
        assert (rl[n] == lse[h, t]) or (math.isinf(rl[n]) and math.isinf(lse[h, t]))


# ----------------------------------------------------------------------------- library routine
def _sdpa_check(fwd, inp):
    """Per sequence, torch's SDPA (float64, CPU) with an additive ALiBi + causal
    bias and enable_gqa; rows that would be empty are skipped (SDPA gives NaN)."""
    F = torch.nn.functional
    out, lse = _run(fwd, inp)
    sq, sk = inp.seqstart_q.tolist(), inp.seqstart_k.tolist()
    ok = True
    for b in range(len(sq) - 1):
        Lq, Lk = sq[b + 1] - sq[b], sk[b + 1] - sk[b]
        if Lq == 0 or Lk == 0:
            continue
        Q = inp.q[sq[b]:sq[b + 1]].double().permute(1, 0, 2)[None]
        K = inp.k[sk[b]:sk[b + 1]].double().permute(1, 0, 2)[None]
        V = inp.v[sk[b]:sk[b + 1]].double().permute(1, 0, 2)[None]
        i = torch.arange(Lq, dtype=torch.float64)[:, None] + (Lk - Lq)
        j = torch.arange(Lk, dtype=torch.float64)[None, :]
        bias = torch.zeros(inp.Hq, Lq, Lk, dtype=torch.float64)
        if inp.alibi_slopes is not None:
            bias = bias - inp.alibi_slopes.double()[:, None, None] * (i - j).abs()[None]
        if inp.causal:
            bias = bias.masked_fill((j > i)[None], float("-inf"))
        live = ~torch.isneginf(bias).all(dim=-1)            # [Hq, Lq]
        ref = F.scaled_dot_product_attention(Q, K, V, attn_mask=bias[None], scale=inp.scale,
                                             enable_gqa=True)[0].permute(1, 0, 2)
        mine = out[sq[b]:sq[b + 1]]
        lv = live.transpose(0, 1)                            # [Lq, Hq]
        if lv.any():
            ok &= (ref[lv] - mine[lv]).abs().max().item() < 1e-12
    return ok


@pytest.mark.parametrize("ci", range(len(TINY_CASES)))
def test_sdpa_library(ci):
    assert _sdpa_check(attention_forward, _tiny(TINY_CASES[ci], seed=100 + ci))


def test_sdpa_library_medium():
    inp = random_case(7, [64, 130, 1, 77], Hq=8, Hkv=2, D=64, dtype="bf16", causal=True,
                      alibi=True)
    assert _sdpa_check(attention_forward, inp)


# ----------------------------------------------------------------------------- closed forms
def test_constant_v():
    inp = random_case(1, [9, 17], Hq=4, Hkv=2, D=8, causal=True, alibi=True)
    c = torch.linspace(-2, 2, 8).half()
    inp.v[:] = c
    out, _ = _run(attention_forward, inp)
    assert (out - c.double()).abs().max().item() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_uniform_weights(causal):
    lq, lk = [6, 3], [10, 3]
    inp = random_case(2, lq, lk, Hq=2, Hkv=1, D=8, causal=causal)
    inp.k[:] = inp.k[0]
    out, lse = _run(attention_forward, inp)
    sq, sk = inp.seqstart_q.tolist(), inp.seqstart_k.tolist()
    for b in range(2):
        for r in range(lq[b]):
            n = min(lk[b], r + (lk[b] - lq[b]) + 1) if causal else lk[b]
            for h in range(2):
                t = sq[b] + r
                qk = math.fsum(float(a) * float(c) for a, c in zip(inp.q[t, h].double(), inp.k[0, 0].double()))
                assert abs(lse[h, t].item() - (inp.scale * qk + math.log(n))) < 1e-12
                mean = inp.v[sk[b]:sk[b] + n, 0].double().mean(0)
                assert (out[t, h] - mean).abs().max().item() < 1e-12


def test_zero_query_causal_alibi_geometric():
    L, m = 23, 0.61
    inp = random_case(4, [L], Hq=1, Hkv=1, D=4, causal=True, alibi=True,
                      slopes=torch.tensor([m], dtype=torch.float32))
    inp.q.zero_()
    m = float(torch.tensor(m, dtype=torch.float32))
    out, lse = _run(attention_forward, inp)
    for r in range(L):
        closed = math.log((1 - math.exp(-m * (r + 1))) / (1 - math.exp(-m)))
        assert abs(lse[0, r].item() - closed) < 1e-12
        w = [math.exp(-m * (r - j)) / math.exp(closed) for j in range(r + 1)]
        ref = [math.fsum(w[j] * float(inp.v[j, 0, d]) for j in range(r + 1)) for d in range(4)]
        assert max(abs(out[r, 0, d].item() - ref[d]) for d in range(4)) < 1e-12


def test_zero_query_noncausal_alibi_two_sided_series():
    L, m = 12, 0.45
    inp = random_case(5, [L], Hq=1, Hkv=1, D=4, alibi=True,
                      slopes=torch.tensor([m], dtype=torch.float32))
    inp.q.zero_()
    m = float(torch.tensor(m, dtype=torch.float32))
    _, lse = _run(attention_forward, inp)
    for r in range(L):
        left = (1 - math.exp(-m * (r + 1))) / (1 - math.exp(-m))
        right = math.exp(-m) * (1 - math.exp(-m * (L - 1 - r))) / (1 - math.exp(-m))
        assert abs(lse[0, r].item() - math.log(left + right)) < 1e-12


def test_zero_slope_is_no_alibi():
    inp = random_case(6, [13, 4], Hq=4, Hkv=2, D=8, causal=True)
    base = _run(attention_forward, inp)
    inp.alibi_slopes = torch.zeros(4)
    zero = _run(attention_forward, inp)
    assert torch.equal(base[0], zero[0]) and torch.equal(base[1], zero[1])


def test_single_key_row():
    # causal: the first row of every sequence sees only its first key
    inp = random_case(8, [5, 9], Hq=2, Hkv=2, D=8, causal=True, alibi=True)
    out, lse = _run(attention_forward, inp)
    for b, t in enumerate(inp.seqstart_q.tolist()[:-1]):
        for h in range(2):
            assert torch.equal(out[t, h], inp.v[t, h].double())
            s = inp.scale * math.fsum(float(a) * float(c) for a, c in zip(inp.q[t, h].double(), inp.k[t, h].double()))
            assert abs(lse[h, t].item() - s) < 1e-12


# ----------------------------------------------------------------------------- invariants
def test_packed_equals_per_sequence():
    inp = random_case(9, [37, 120, 8, 200], Hq=8, Hkv=8, D=16, causal=True, alibi=True)
    out, lse = _run(attention_forward, inp)
    sq = inp.seqstart_q.tolist()
    for b in range(4):
        s = slice(sq[b], sq[b + 1])
        L = sq[b + 1] - sq[b]
        o1, l1 = attention_forward(inp.q[s], inp.k[s], inp.v[s], [0, L], [0, L], causal=True,
                                   alibi_slopes=inp.alibi_slopes, scale=inp.scale)
        assert torch.equal(o1, out[s]) and torch.equal(l1, lse[:, s])


def test_segment_permutation_permutes_output():
    lens = [7, 3, 12]
    inp = random_case(10, lens, Hq=4, Hkv=2, D=8, causal=True, alibi=True)
    out, lse = _run(attention_forward, inp)
    sq = inp.seqstart_q.tolist()
    perm = [2, 0, 1]
    cat = lambda x: torch.cat([x[sq[b]:sq[b + 1]] for b in perm])
    ss = seqstart_from_lengths([lens[b] for b in perm])
    o2, l2 = attention_forward(cat(inp.q), cat(inp.k), cat(inp.v), ss, ss, causal=True,
                               alibi_slopes=inp.alibi_slopes, scale=inp.scale)
    assert torch.equal(o2, cat(out))
    assert torch.equal(l2, torch.cat([lse[:, sq[b]:sq[b + 1]] for b in perm], dim=1))


@pytest.mark.parametrize("Hkv", [1, 2, 4])
def test_gqa_equals_mha_after_repeat_interleave(Hkv):
    Hq = 8
    inp = random_case(11, [19, 33], Hq=Hq, Hkv=Hkv, D=16, causal=True, alibi=True)
    out, lse = _run(attention_forward, inp)
    k_rep = inp.k.repeat_interleave(Hq // Hkv, dim=1)
    v_rep = inp.v.repeat_interleave(Hq // Hkv, dim=1)
    o2, l2 = attention_forward(inp.q, k_rep, v_rep, inp.seqstart_q, inp.seqstart_k, causal=True,
                               alibi_slopes=inp.alibi_slopes, scale=inp.scale)
    assert (out - o2).abs().max().item() < 1e-13 and (lse - l2).abs().max().item() < 1e-13


def test_mqa_is_gqa1_broadcast():
    inp = random_case(12, [21], Hq=4, Hkv=1, D=8)
    out, _ = _run(attention_forward, inp)
    for h in range(4):
        oh, _ = attention_forward(inp.q[:, h:h + 1], inp.k, inp.v, inp.seqstart_q, inp.seqstart_k,
                                  scale=inp.scale)
        assert torch.equal(oh[:, 0], out[:, h])


def test_causal_mask_is_lower_triangular():
    L = 14
    inp = random_case(13, [L], Hq=2, Hkv=1, D=8, causal=True)
    out, _ = _run(attention_forward, inp)
    # explicit tril mask through plain softmax
    for h in range(2):
        S = inp.scale * (inp.q[:, h].double() @ inp.k[:, 0].double().T)
        S = S.masked_fill(torch.tril(torch.ones(L, L, dtype=torch.bool)).logical_not(), float("-inf"))
        ref = torch.softmax(S, dim=1) @ inp.v[:, 0].double()
        assert (ref - out[:, h]).abs().max().item() < 1e-13


def test_future_keys_do_not_change_a_row():
    L = 20
    inp = random_case(14, [L], Hq=2, Hkv=2, D=8, causal=True, alibi=True)
    out, lse = _run(attention_forward, inp)
    for r in [0, 5, 13]:
        inp2 = random_case(14, [L], Hq=2, Hkv=2, D=8, causal=True, alibi=True)
        inp2.k[r + 1:] = torch.randn_like(inp2.k[r + 1:].float()).half()
        inp2.v[r + 1:] = 100.0
        o2, l2 = _run(attention_forward, inp2)
        assert torch.equal(o2[: r + 1], out[: r + 1]) and torch.equal(l2[:, : r + 1], lse[:, : r + 1])
        assert not torch.equal(o2[r + 1:], out[r + 1:])


@pytest.mark.parametrize("Lq", [1, 6])
def test_split_kv_lse_combine_identity(Lq):
    """Splitting the keys of one sequence into chunks and merging the chunk
    results by their log-sum-exp gives the unsplit result (no mask, no ALiBi:
    the chunk results do not depend on key positions)."""
    Lk = 57
    inp = random_case(15, [Lq], [Lk], Hq=4, Hkv=2, D=8)
    out, lse = _run(attention_forward, inp)
    rnd = random.Random(0)
    cuts = sorted(rnd.sample(range(1, Lk), 4))
    bounds = [0] + cuts + [Lk]
    parts = []
    for c0, c1 in zip(bounds[:-1], bounds[1:]):
        parts.append(attention_forward(inp.q, inp.k[c0:c1], inp.v[c0:c1], [0, Lq], [0, c1 - c0],
                                       scale=inp.scale))
    L = torch.logsumexp(torch.stack([p[1] for p in parts]), dim=0)           # [Hq, Lq]
    merged = sum(torch.exp(p[1] - L).transpose(0, 1)[..., None] * p[0] for p in parts)
    assert (L - lse).abs().max().item() < 1e-12
    assert (merged - out).abs().max().item() < 1e-12


def test_decode_equals_last_prefill_row():
    """One query at the end of a sequence (the decode case) sees the whole KV
    history with ALiBi distances counted from its own position."""
    L = 31
    inp = random_case(16, [L], Hq=4, Hkv=2, D=16, causal=True, alibi=True)
    out, lse = _run(attention_forward, inp)
    for causal in (True, False):
        od, ld = attention_forward(inp.q[L - 1:L], inp.k, inp.v, [0, 1], [0, L], causal=causal,
                                   alibi_slopes=inp.alibi_slopes, scale=inp.scale)
        assert (od[0] - out[L - 1]).abs().max().item() < 1e-13
        assert (ld[:, 0] - lse[:, L - 1]).abs().max().item() < 1e-13


def test_workload_generator_lengths_and_slopes():
    """The long-sequence workloads draw the lengths the design notes quote."""
    w4 = generate("varlen_causal_gqa_64seq_h32kv8_d128_bf16", num_seqs=2)
    from mea_workloads import _lengths, get_workload
    lq, lk = _lengths(get_workload("varlen_causal_gqa_64seq_h32kv8_d128_bf16"), 0)
    assert (sum(lq), min(lq), max(lq)) == (137663, 138, 4085) and lq == lk
    lq, lk = _lengths(get_workload("decode_splitkv_64req_h64kv8_d128_bf16"), 0)
    assert lq == [1] * 64 and (sum(lk), min(lk), max(lk)) == (1101299, 1110, 32680)
    s = alibi_slopes(32)
    import numpy as np
    assert s[0].item() == float(np.float32(2.0 ** -0.25)) and s[-1].item() == 2.0 ** -8
    assert w4.q.shape[0] == sum(lq[:0]) + w4.seqlens_q[0] + w4.seqlens_q[1]


# ----------------------------------------------------------------------------- mutation tests
MUTATIONS = [
    ("g = h // per_group", "g = h % Hkv"),                                   # wrong head grouping
    ("S = S - slope *", "S = S + slope *"),                                  # ALiBi sign
    ("if slope is not None:", "if False:"),                                  # dropped ALiBi
    ("kpos[None, :] > qpos[:, None]", "kpos[None, :] >= qpos[:, None]"),     # causal off by one
    ("+ (L_k - L_q)", "+ 0"),                                                # top-left alignment
    ("S = scale * (Q @ K.transpose(0, 1))", "S = (Q @ K.transpose(0, 1))"),  # dropped scale
    ("lse = torch.logsumexp(S, dim=1)", "lse = torch.logsumexp(S, dim=1) / math.log(2)"),  # log base
    ("out = P @ V", "out = P @ V.flip(0)"),                                  # V rows misaligned
    ("V64[sk[b]:sk[b + 1], g, :]", "V64[sk[b]:sk[b + 1], 0, :]"),            # V head index
    ("(qpos[:, None] - kpos[None, :]).abs()", "(qpos[:, None] - kpos[None, :])"),  # |.| dropped
    ("K64[sk[b]:sk[b + 1], g, :]", "K64[sq[b]:sq[b] + (sk[b + 1] - sk[b]), g, :]"),  # q offsets for k
]


def _mutant(old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) >= 1, old
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["math"] = math
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod.attention_forward


def _pins_pass(fwd):
    for ci, case in enumerate(TINY_CASES):
        inp = _tiny(case, seed=200 + ci)
        try:
            out, lse = _run(fwd, inp)
        except Exception:
            return False
        bo, bl = brute_force(inp.q, inp.k, inp.v, inp.seqstart_q, inp.seqstart_k, inp.causal,
                             inp.alibi_slopes, inp.scale)
        if not (_same(out, bo, 1e-12) and _same(lse, bl, 1e-12)):
            return False
    return True


def test_unmutated_oracle_passes_pins():
    assert _pins_pass(attention_forward)


@pytest.mark.parametrize("mi", range(len(MUTATIONS)))
def test_planted_mistake_fails_pins(mi):
    old, new = MUTATIONS[mi]
    assert not _pins_pass(_mutant(old, new))
