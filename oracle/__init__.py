"""CPU fp64 oracle for the forward-mode JVP of masked scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP path (``attention_jvp_causal_attn_amd``) and imports nothing from it.

Sources (page titles as they appear on the web pages this method is taken from):

* "Causal-rCM: A Unified Teacher-Forcing and Self-Forcing Open Recipe for
  Autoregressive Diffusion Distillation ..." (paperlayer.ai summary of
  arXiv 2606.25473), Appendix B "FlashAttention-2 JVP Kernel with Custom Masks"
  and Section 3 (continuous-time consistency, the TF-masked packed forward).
* "Causal Forcing: Autoregressive Diffusion Distillation Done Right ..."
  (paperlayer.ai summary of arXiv 2602.02214), Section 2 Background (teacher
  forcing concatenates clean and noisy videos under a causal attention mask).

Every function states the passage it follows.  Pins (tests that tie the oracle
to something other than itself) live in ``tests/test_oracle_pins.py``.
"""

from .masks import (  # noqa: F401
    tf_allowed,
    dense_allowed,
    rects_allowed,
    block_causal_allowed,
)
from .attn_jvp import masked_attention, masked_attention_jvp  # noqa: F401
from .attn_bwd import masked_attention_grad  # noqa: F401
