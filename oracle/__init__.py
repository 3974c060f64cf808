"""CPU float64 oracle for the fused attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The GPU product path
never routes through it, and it shares no code with the HIP library or its
Python binding (the seeded input generators in ``mea_workloads`` are the only
code both sides use, and they hold none of the attention arithmetic).

What it computes is the plain definition of attention over packed
variable-length sequences, its gradients, its fp8-input form, and the SwiGLU
feed-forward layer of the same transformer block (``oracle.ffn``); see ``oracle.attention`` for the definition and the
passages of the pages it follows.  Every function here is pinned by
``tests/test_oracle.py`` (brute force, closed forms, invariants and a library
routine) except the readings listed as "parity unpinned" in
``oracle.attention``'s module docstring.
"""
from .attention import (attention_backward, attention_backward_scales, attention_forward,
                        attention_forward_fp8, attention_rows)
from .ffn import silu, swiglu_ffn, swiglu_ffn_rows

__all__ = ["attention_forward", "attention_rows", "attention_backward", "attention_backward_scales",
           "attention_forward_fp8", "silu",
           "swiglu_ffn", "swiglu_ffn_rows"]
