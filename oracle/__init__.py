"""Plain float64 CPU oracle of the Lizard hybrid attention layer.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP
library and its Python binding) never imports or calls it and shares no
code with it.

Source: "Lizard: An Efficient Linearization Framework for Large Language
Models" (arXiv 2507.09025) as explained on gist.science (German, Italian and
Portuguese pages), shd-paper.top and chatpaper.ai.  The pages give the gate
(a sigmoid of a projection), the hybrid sum Y = Y_gate + alpha * Y_anchor,
a data-adaptive recurrence with constant-size state, and a sliding window
with meta-memory sink tokens that do not contribute values.  The exact
recurrence, window extent, softmax scale and sink semantics they leave open
are fixed by the readings listed in the module docstring of
``oracle.lizard``.
"""
from .lizard import (  # noqa: F401
    gla_recurrent,
    gla_quadratic,
    gla_chunked,
    anchor_window,
    anchor_bruteforce,
    lizard_fwd,
    lizard_decode_step,
    lizard_bwd,
    gla_bwd_recurrent,
    anchor_bwd,
    log_sigmoid,
    lizard_fwd_logit,
    lizard_bwd_logit,
    lizard_decode_step_logit,
    lizard_fwd_continue,
    softmax_attention_causal,
    transfer_loss,
    stage1_step,
)
