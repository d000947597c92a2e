"""CPU oracle for exact attention -- TEST INFRASTRUCTURE, not product code.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from here. The HIP library never calls it
and shares no code with it.

Everything here is the plain definition of scaled-dot-product attention and
its analytic gradient, evaluated in float64 over the bf16 input bits
(see ``oracle.attention`` for the passages each function follows), and in
``oracle.dropout`` the same with attention dropout (a Philox4x32-10 keep
mask on the probabilities).
"""
from .attention import (  # noqa: F401
    widen_bf16,
    keep_matrix,
    head_forward,
    head_backward,
    head_grad_rows,
    head_grad_cols,
    attn_fwd_ref,
    attn_bwd_ref,
    online_softmax_ref,
    naive_bruteforce,
    naive_bruteforce_bits,
)
