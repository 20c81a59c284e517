"""CPU oracle for the fused attention forward pass and its gradients.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import anything from this package; the product path (the HIP library and its Python binding)
never does, and the two share no code.

Everything here is plain float64 NumPy (or pure Python for the tiny brute-force case) written from
the five pages on tiled/online-softmax attention:
  * "SDPA and FlashAttention's tiling" (octlm notes),
  * "Explain tiled attention and verify its output" (aiml.sh lab),
  * "4.2 FlashAttention I: IO-Awareness & The Online Softmax" (LLM stack book),
  * "Attention from scratch + roofline" (LLM systems cookbook),
  * "Efficient attention & KV cache" (ML interview book).

Parity status: every function below is pinned by `tests/test_oracle_pins.py`,
`tests/test_window_pins.py`, `tests/test_backward_pins.py`, `tests/test_paged_pins.py`,
`tests/test_varlen_pins.py` and `tests/test_accounting.py` against
values the pages print, closed forms, invariants, finite differences and library special cases.
No function is "parity unpinned".
"""

from .attention import (  # noqa: F401
    brute_attention,
    dense_attention,
    dense_head,
    merge_partials,
    online_logsumexp_trace,
    stream_softmax,
    stream_weighted_sum,
    tiled_attention,
    tiled_head,
)
from .backward import (  # noqa: F401
    backward_cols,
    backward_flops,
    backward_rows,
    dense_backward,
    dense_backward_head,
    loss_gradient_fd,
    tiled_backward,
    tiled_backward_head,
)
from .paged import gather_sequence, paged_decode  # noqa: F401
from .varlen import varlen_attention, varlen_backward  # noqa: F401
from . import accounting  # noqa: F401
