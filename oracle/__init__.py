"""fp64 CPU oracle for Shifted Sparse Attention (S2-Attn) and for the
LoRA-adapted q/k/v projections ahead of it.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it; the only module both sides use is the
seeded input generator ``workloads.py``, which holds none of the method's
arithmetic.

Every function here is pinned by the CPU tests in ``tests/test_oracle_*.py``
against closed forms, invariants, brute force, library routines and the
values the pages print.
"""
from .s2attn_ref import (  # noqa: F401
    head_shift,
    kv_head,
    roll_sequence,
    rope_angles,
    rope_rotate,
    group_causal_attention,
    group_causal_attention_backward,
    s2attn_forward,
    s2attn_backward,
    s2attn_unit_forward,
    s2attn_unit_backward,
    head_unit_forward,
    head_unit_backward,
    unit_positions,
    dense_causal_attention,
    brute_force_masked_attention,
)
from .lora_qkv_ref import (  # noqa: F401
    lora_projection,
    lora_qkv_forward,
    lora_qkv_backward,
)
