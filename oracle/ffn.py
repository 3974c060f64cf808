"""Plain float64 SwiGLU feed-forward layer (CPU oracle).

TEST INFRASTRUCTURE ONLY: imported by the tests, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product path.

Source: "How to Build Memory-Efficient Transformers with xFormers Using Packed
Sequences, GQA, ALiBi, SwiGLU, and Causal Attention" (yifor-blog),
optimisation item 4: the feed-forward layers of the tutorial's transformer use
the SwiGLU activation in place of ReLU or GELU.  The page gives no formula;
the reading taken is the gated linear unit with the SiLU (swish) gate:

  hidden[t, f] = SiLU(sum_i x[t, i] w_gate[f, i]) * sum_i x[t, i] w_up[f, i]
  out[t, j]    = sum_f hidden[t, f] w_down[j, f]
  SiLU(z)      = z / (1 + exp(-z))

with the weights in a linear layer's [out_features, in_features] layout.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import torch

__all__ = ["silu", "swiglu_ffn", "swiglu_ffn_rows"]


def silu(z: torch.Tensor) -> torch.Tensor:
    """z * sigmoid(z), written out."""
    return z / (1.0 + torch.exp(-z))


def _f64(x: torch.Tensor) -> torch.Tensor:
    return x.detach().to("cpu").to(torch.float64)


def swiglu_ffn(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor,
               w_down: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Returns float64 (hidden [T, d_ff], out [T, d_model], out_abs [T, d_model])
    where out_abs = sum_f |hidden[t, f] w_down[j, f]|, the scale of the terms of
    each output element (for error bounds)."""
    X, Wg, Wu, Wd = _f64(x), _f64(w_gate), _f64(w_up), _f64(w_down)
    gate = X @ Wg.transpose(0, 1)
    up = X @ Wu.transpose(0, 1)
    hidden = silu(gate) * up
    out = hidden @ Wd.transpose(0, 1)
    out_abs = hidden.abs() @ Wd.abs().transpose(0, 1)
    return hidden, out, out_abs


def swiglu_ffn_rows(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                    rows: Sequence[int]) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """The same for the selected token rows only (sampled checks at full size)."""
    idx = torch.as_tensor(list(rows), dtype=torch.long)
    return swiglu_ffn(x[idx], w_gate, w_up, w_down)
