"""Plain float64 attention over packed variable-length sequences (CPU oracle).

TEST INFRASTRUCTURE ONLY: imported by the tests, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product path.

Sources (web pages; section names as printed on them):
  [P1] "Cómo construir transformadores con memoria eficiente con xFormers usando
       secuencias empaquetadas, GQA, ALiBi, SwiGLU y atención causal"
       (7minutos.es) -- section 4, packed variable-length batch with
       BlockDiagonalMask / BlockDiagonalCausalMask; section 5, grouped-query
       attention in the 5-D BMGHK layout.
  [P2] "How to Build Memory-Efficient Transformers with xFormers Using Packed
       Sequences, GQA, ALiBi, SwiGLU, and Causal Attention" (yifor-blog) --
       optimisation items 1 (packed sequences + block-diagonal mask), 2 (GQA),
       3 (ALiBi: a different additive linear position penalty per head) and
       5 (causal attention: implicit lower-triangular mask).
  [P3] "multi query attention代码" (cidian.kuaisou.com) -- the self-attention
       snippet: scores = Q K^T / sqrt(d_k), softmax, weighted sum of V.
  [P4] "大模型推理加速终极指南：xformers如何让Transformer性能飙升300%"
       (zizhi168.cn) -- section 3, mixed-precision pipeline (FP16/BF16/FP8).
  [P5] "group query attention gqa" (cidian.kuaisou.com) -- GQA-G definition
       (G groups, each sharing one K/V head; GQA-1 = MQA, GQA-H = MHA) and the
       check that SDPA with enable_gqa equals SDPA after repeat_interleave of
       the K/V heads along the head axis.

Definition computed (for every sequence b and query head h):
  L_q, L_k = lengths of sequence b; off = L_k - L_q;
  g = h // (Hq // Hkv)                                     [P5; P1 section 5]
  S[r, j] = scale * sum_d q[sq_b + r, h, d] * k[sk_b + j, g, d]      [P3]
  with ALiBi:   S[r, j] -= slope_h * |(r + off) - j|              [P2 item 3]
  with causal:  S[r, j] = -inf where j > r + off                  [P2 item 5]
  keys of other sequences never enter row r            [P1 section 4; P2 item 1]
  lse[h, sq_b + r] = ln sum_j exp(S[r, j])   (-inf for a row with no key)
  out[sq_b + r, h, :] = sum_j exp(S[r, j] - lse) v[sk_b + j, g, :]  (0 if empty)

Readings where the pages are silent (each is listed in the design notes):
  * scale is applied to Q K^T before the bias is added, and the bias is not
    scaled;
  * ALiBi positions are local to each sequence; the penalty is
    slope * distance, slopes given per query head;
  * when L_q != L_k, query row r sits at key position r + off (queries are the
    last L_q positions of the sequence; a single decode query sees its whole
    KV history);
  * a row with no allowed key has out = 0 and lse = -inf;
  * lse is the natural-log normaliser of the scaled, biased, masked scores.
Parity unpinned by the pages: the ALiBi slope values (an input here), the
non-causal |i - j| form of ALiBi, the L_q != L_k causal alignment beyond the
decode == last-prefill-row identity, and the empty-row convention.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import torch

__all__ = ["attention_forward", "attention_rows", "attention_backward", "attention_backward_scales",
           "attention_forward_fp8"]


def _f64(x: torch.Tensor) -> torch.Tensor:
    """Exact upcast of the given fp16/bf16/fp32 values to float64 on the CPU."""
    return x.detach().to("cpu").to(torch.float64)


def _starts(seqstart) -> List[int]:
    return [int(s) for s in (seqstart.tolist() if torch.is_tensor(seqstart) else seqstart)]


def _softmax_block(Q: torch.Tensor, K: torch.Tensor, qpos: torch.Tensor, causal: bool,
                   slope: Optional[float], scale: float) -> Tuple[torch.Tensor, torch.Tensor]:
    """Softmax weights P [R, L_k] and lse [R] of query rows Q [R, D] (at key
    positions qpos [R]) over one sequence's keys K [L_k, D]."""
    L_k = K.shape[0]
    kpos = torch.arange(L_k, dtype=torch.float64)
    S = scale * (Q @ K.transpose(0, 1))                       # [P3]: scaled scores
    if slope is not None:                                      # [P2 item 3]: ALiBi
        S = S - slope * (qpos[:, None] - kpos[None, :]).abs()
    if causal:                                                 # [P2 item 5]
        S = S.masked_fill(kpos[None, :] > qpos[:, None], float("-inf"))
    if L_k == 0:
        lse = torch.full((Q.shape[0],), float("-inf"), dtype=torch.float64)
    else:
        lse = torch.logsumexp(S, dim=1)
    empty = torch.isneginf(lse)
    P = torch.exp(S - torch.where(empty, 0.0, lse)[:, None])  # softmax weights
    P = torch.where(empty[:, None], 0.0, P)
    return P, lse


def _one_row_block(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, qpos: torch.Tensor,
                   causal: bool, slope: Optional[float], scale: float
                   ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention of query rows Q [R, D] (at key positions qpos [R]) over one
    sequence's keys K, V [L_k, D].  Returns out [R, D] and lse [R]."""
    P, lse = _softmax_block(Q, K, qpos, causal, slope, scale)
    out = P @ V
    return out, lse


def attention_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      seqstart_q, seqstart_k, *, causal: bool = False,
                      alibi_slopes: Optional[torch.Tensor] = None,
                      scale: Optional[float] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Reference forward over packed sequences.

    q [Tq, Hq, D], k and v [Tk, Hkv, D] (any float dtype, upcast exactly);
    seqstart_q / seqstart_k: n+1 non-decreasing offsets starting at 0.
    Returns out float64 [Tq, Hq, D] and lse float64 [Hq, Tq].  ``scale`` None
    means 1/sqrt(D) [P3].  Slopes are taken at their given (float32) values.
    """
    Q64, K64, V64 = _f64(q), _f64(k), _f64(v)
    Tq, Hq, D = Q64.shape
    Tk, Hkv, Dk = K64.shape
    assert Dk == D and tuple(V64.shape) == (Tk, Hkv, D) and Hq % Hkv == 0
    if scale is None:
        scale = D ** -0.5
    slopes = None if alibi_slopes is None else [float(s) for s in _f64(alibi_slopes)]
    sq, sk = _starts(seqstart_q), _starts(seqstart_k)
    assert len(sq) == len(sk)
    per_group = Hq // Hkv
    out = torch.zeros((Tq, Hq, D), dtype=torch.float64)
    lse = torch.full((Hq, Tq), float("-inf"), dtype=torch.float64)
    for b in range(len(sq) - 1):
        L_q, L_k = sq[b + 1] - sq[b], sk[b + 1] - sk[b]
        if L_q == 0:
            continue
        qpos = torch.arange(L_q, dtype=torch.float64) + (L_k - L_q)
        for h in range(Hq):
            g = h // per_group                                  # [P5]: head grouping
            o, l = _one_row_block(Q64[sq[b]:sq[b + 1], h, :], K64[sk[b]:sk[b + 1], g, :],
                                  V64[sk[b]:sk[b + 1], g, :], qpos, causal,
                                  None if slopes is None else slopes[h], float(scale))
            out[sq[b]:sq[b + 1], h, :] = o
            lse[h, sq[b]:sq[b + 1]] = l
    return out, lse


def attention_rows(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seqstart_q, seqstart_k,
                   rows: Sequence[Tuple[int, int]], *, causal: bool = False,
                   alibi_slopes: Optional[torch.Tensor] = None,
                   scale: Optional[float] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The same definition evaluated for selected (packed token, query head)
    rows only, for sampled checks on inputs too large to do whole.
    Returns out float64 [len(rows), D] and lse float64 [len(rows)]."""
    Tq, Hq, D = q.shape
    Tk, Hkv, _ = k.shape
    if scale is None:
        scale = D ** -0.5
    sq, sk = _starts(seqstart_q), _starts(seqstart_k)
    per_group = Hq // Hkv
    outs = torch.zeros((len(rows), D), dtype=torch.float64)
    lses = torch.full((len(rows),), float("-inf"), dtype=torch.float64)
    for n, (t, h) in enumerate(rows):
        b = max(i for i in range(len(sq) - 1) if sq[i] <= t < sq[i + 1])
        L_q, L_k = sq[b + 1] - sq[b], sk[b + 1] - sk[b]
        g = h // per_group
        qpos = torch.tensor([t - sq[b] + (L_k - L_q)], dtype=torch.float64)
        slope = None if alibi_slopes is None else float(_f64(alibi_slopes)[h])
        o, l = _one_row_block(_f64(q[t:t + 1, h, :]), _f64(k[sk[b]:sk[b + 1], g, :]),
                              _f64(v[sk[b]:sk[b + 1], g, :]), qpos, causal, slope, float(scale))
        outs[n] = o[0]
        lses[n] = l[0]
    return outs, lses


def attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor,
                       seqstart_q, seqstart_k, *, causal: bool = False,
                       alibi_slopes: Optional[torch.Tensor] = None,
                       scale: Optional[float] = None
                       ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Gradients of sum(out * dout) with respect to q, k and v, for the
    forward that ``attention_forward`` computes.

    The pages time the backward pass of the same attention beside the
    forward ([P2], the performance comparison of xFormers against standard
    attention) and train a GPT-style model with it; they give no formulas, so
    this is the derivative of the definition written out by the chain rule,
    per sequence b and query head h with g = h // (Hq / Hkv):
      P   = softmax weights of the forward (zero rows where no key is allowed)
      dV_g += P^T dO_h                          (out = P V)
      dP  = dO_h V_g^T
      dS  = P * (dP - rowsum(P * dP))           (Jacobian of a row softmax)
      dQ_h  = scale * dS K_g
      dK_g += scale * dS^T Q_h                  (S = scale Q K^T + bias)
    The sums over the query heads of one group give the K/V gradients of the
    shared head [P5].  The ALiBi slopes, the causal mask and the block-diagonal
    mask are constants: no gradient flows to them.
    Returns dq float64 [Tq, Hq, D], dk and dv float64 [Tk, Hkv, D].
    """
    Q64, K64, V64, dO64 = _f64(q), _f64(k), _f64(v), _f64(dout)
    Tq, Hq, D = Q64.shape
    Tk, Hkv, _ = K64.shape
    assert tuple(dO64.shape) == (Tq, Hq, D) and Hq % Hkv == 0
    if scale is None:
        scale = D ** -0.5
    slopes = None if alibi_slopes is None else [float(s) for s in _f64(alibi_slopes)]
    sq, sk = _starts(seqstart_q), _starts(seqstart_k)
    per_group = Hq // Hkv
    dq = torch.zeros((Tq, Hq, D), dtype=torch.float64)
    dk = torch.zeros((Tk, Hkv, D), dtype=torch.float64)
    dv = torch.zeros((Tk, Hkv, D), dtype=torch.float64)
    for b in range(len(sq) - 1):
        L_q, L_k = sq[b + 1] - sq[b], sk[b + 1] - sk[b]
        if L_q == 0 or L_k == 0:
            continue
        qpos = torch.arange(L_q, dtype=torch.float64) + (L_k - L_q)
        for h in range(Hq):
            g = h // per_group
            Qh = Q64[sq[b]:sq[b + 1], h, :]
            Kg = K64[sk[b]:sk[b + 1], g, :]
            Vg = V64[sk[b]:sk[b + 1], g, :]
            dOh = dO64[sq[b]:sq[b + 1], h, :]
            P, _ = _softmax_block(Qh, Kg, qpos, causal, None if slopes is None else slopes[h],
                                  float(scale))
            dv[sk[b]:sk[b + 1], g, :] += P.transpose(0, 1) @ dOh
            dP = dOh @ Vg.transpose(0, 1)
            dS = P * (dP - (P * dP).sum(dim=1, keepdim=True))
            dq[sq[b]:sq[b + 1], h, :] = scale * (dS @ Kg)
            dk[sk[b]:sk[b + 1], g, :] += scale * (dS.transpose(0, 1) @ Qh)
    return dq, dk, dv


def attention_backward_scales(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor,
                              seqstart_q, seqstart_k, *, causal: bool = False,
                              alibi_slopes: Optional[torch.Tensor] = None,
                              scale: Optional[float] = None, floor: float = 0.0
                              ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Error scales of the gradients: for every element of dq, dk and dv, the
    sum of the absolute values of the terms ``attention_backward`` adds up for
    it, for element-wise error bounds (not part of the method).

    An implementation that rounds the softmax weights P and dS to a 16-bit
    type with unit roundoff u, and forms rowsum(dO * out) from a rounded out,
    errs on each term by at most u times that term's size, taking P and |dS|
    no smaller than ``floor`` (the smallest normal number of the type: below
    it a rounding errs by up to u * floor) on allowed (query, key) pairs.
    With p = max(P, floor) and d = max(|dS|, floor) there, 0 on masked pairs,
    and E_i = sum_d |dO[i, d] out[i, d]| (the size of the row term):
      av_g += p^T |dO_h|
      aq_h  = scale * (d |K_g| + (p * E) |K_g|)
      ak_g += scale * (d^T |Q_h| + (p * E)^T |Q_h|)
    Returns float64 (aq [Tq, Hq, D], ak [Tk, Hkv, D], av [Tk, Hkv, D]).
    """
    Q64, K64, V64, dO64 = _f64(q), _f64(k), _f64(v), _f64(dout)
    Tq, Hq, D = Q64.shape
    Tk, Hkv, _ = K64.shape
    if scale is None:
        scale = D ** -0.5
    slopes = None if alibi_slopes is None else [float(s) for s in _f64(alibi_slopes)]
    sq, sk = _starts(seqstart_q), _starts(seqstart_k)
    per_group = Hq // Hkv
    aq = torch.zeros((Tq, Hq, D), dtype=torch.float64)
    ak = torch.zeros((Tk, Hkv, D), dtype=torch.float64)
    av = torch.zeros((Tk, Hkv, D), dtype=torch.float64)
    for b in range(len(sq) - 1):
        L_q, L_k = sq[b + 1] - sq[b], sk[b + 1] - sk[b]
        if L_q == 0 or L_k == 0:
            continue
        qpos = torch.arange(L_q, dtype=torch.float64) + (L_k - L_q)
        kpos = torch.arange(L_k, dtype=torch.float64)
        allowed = torch.ones((L_q, L_k), dtype=torch.bool)
        if causal:
            allowed = kpos[None, :] <= qpos[:, None]
        for h in range(Hq):
            g = h // per_group
            Qh = Q64[sq[b]:sq[b + 1], h, :]
            Kg = K64[sk[b]:sk[b + 1], g, :]
            Vg = V64[sk[b]:sk[b + 1], g, :]
            dOh = dO64[sq[b]:sq[b + 1], h, :]
            P, _ = _softmax_block(Qh, Kg, qpos, causal, None if slopes is None else slopes[h],
                                  float(scale))
            dP = dOh @ Vg.transpose(0, 1)
            dS = P * (dP - (P * dP).sum(dim=1, keepdim=True))
            E = (dOh * (P @ Vg)).abs().sum(dim=1, keepdim=True)
            live = allowed & (P.sum(dim=1, keepdim=True) > 0)       # rows with no key stay 0
            p = torch.where(live, P.clamp_min(floor), 0.0)
            d = torch.where(live, dS.abs().clamp_min(floor), 0.0)
            av[sk[b]:sk[b + 1], g, :] += p.transpose(0, 1) @ dOh.abs()
            aq[sq[b]:sq[b + 1], h, :] = scale * ((d + p * E) @ Kg.abs())
            ak[sk[b]:sk[b + 1], g, :] += scale * ((d + p * E).transpose(0, 1) @ Qh.abs())
    return aq, ak, av


def attention_forward_fp8(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, q_scale: float,
                          k_scale: float, v_scale: float, seqstart_q, seqstart_k, *,
                          causal: bool = False, alibi_slopes: Optional[torch.Tensor] = None,
                          scale: Optional[float] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The forward on 8-bit inputs with per-tensor scales.

    [P4] section 3 lists FP8 among the formats of the mixed-precision attention
    pipeline.  The tensors hold OCP e4m3 codes (torch.float8_e4m3fn; the
    decoding is pinned against the format's definition in the tests) and the
    values meant are scale * code: q = q_scale * q8, k = k_scale * k8,
    v = v_scale * v8, each formed exactly in float64, then the same definition
    as ``attention_forward``.
    """
    q = _f64(q8) * float(q_scale)
    k = _f64(k8) * float(k_scale)
    v = _f64(v8) * float(v_scale)
    return attention_forward(q, k, v, seqstart_q, seqstart_k, causal=causal,
                             alibi_slopes=alibi_slopes, scale=scale)
