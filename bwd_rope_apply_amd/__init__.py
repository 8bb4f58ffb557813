"""Exact causal softmax attention with rotary position embedding and
learnable log-frequencies (forward and backward, including d alpha) on AMD
MI355X (gfx950), behind the C ABI of ``include/rope_attn.h``.

Also Gram-threshold token selection and its cascade step
(``include/gram_select.h``).

``rope_attn_fwd`` / ``rope_attn_bwd`` (also ``fwd`` / ``bwd``; they take
the stage bits and options of the ``_ex`` entry points as keywords),
``gram_select`` and ``gram_cascade`` are thin ctypes wrappers over
``librope_attn.so``; build it with ``python -m bwd_rope_apply_amd.build``.
``workloads`` draws the seeded synthetic inputs.
"""
from ._lib import fwd, bwd, load, workspace_bytes, workspace_flags, RopeAttnError, FP32, BF16  # noqa: F401
from ._lib import gram_select, gram_cascade  # noqa: F401

rope_attn_fwd = fwd
rope_attn_bwd = bwd
