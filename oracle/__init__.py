"""CPU oracle for exact attention, forward and backward (test infrastructure only).

This package is the reference that the GPU path is checked against. It is plain,
slow and meant to be read against the pages line by line: float64 NumPy, the
three-pass softmax with the score matrix S and the probability matrix P written
out in full, and a dense Hadamard matrix for the FP8 pre-rotation.

Only the test suite, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import it. The product path (the HIP library and its
Python binding) never imports, calls or links anything here, and this package
shares no code, tables or constants with it.

Modules
-------
attention  three-pass attention (S, P, O, LSE), the streaming online-softmax
           recurrence and the two-state merge, used to pin the three-pass form.
e4m3       the OCP FP8 E4M3 (1-4-3, bias 7, max 448) codec, round to nearest
           even with saturation.
hadamard   the normalised Sylvester Hadamard matrix and the random-sign
           incoherent rotation x -> x H D.
fp8        per-64-row block quantisation and the two FP8 reference results
           (O_true on the original inputs, O_deq on the dequantised ones).
attention_bwd
           the closed-form gradients dQ, dK, dV (P rebuilt from L, D = rowsum(dO o O),
           dS = P o (dP - D)), materialised for short rows or sampled for long ones.
"""

from .attention import (  # noqa: F401
    attention_fp64,
    attention_probs_fp64,
    online_softmax_attention,
    merge_states,
)
from .e4m3 import e4m3_decode, e4m3_encode, E4M3_MAX  # noqa: F401
from .hadamard import sylvester_hadamard, incoherent_rotate  # noqa: F401
from .fp8 import block_quantize, block_dequantize, fp8_reference  # noqa: F401
