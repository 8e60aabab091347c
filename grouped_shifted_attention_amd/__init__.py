"""MI355X-native Shifted Sparse Attention (S2-Attn, LongLoRA).

The compute lives in libs2attn.so (hand-written HIP kernels for gfx950 behind
the C ABI in include/s2attn.h); this package only marshals torch tensors to
it.  Build the library with ``python -m grouped_shifted_attention_amd.build``.
"""
from .flops import (  # noqa: F401
    s2attn_fwd_flops,
    s2attn_bwd_flops,
    fwd_algorithmic_bytes,
    bwd_algorithmic_bytes,
)
from .ops import (  # noqa: F401
    S2AttnFunction,
    s2attn,
    s2attn_bwd,
    s2attn_bwd_dkdv,
    s2attn_bwd_dq,
    s2attn_bwd_preprocess,
    bwd_workspace,
    s2attn_bwd_rope,
    s2attn_fwd,
    s2attn_fwd_rope,
    s2attn_workspace_sizes,
    s2attn_lora_qkv_fwd,
    lora_qkv_workspace,
    s2attn_lora_qkv_bwd,
    lora_qkv_bwd_workspace,
    LoraQKVFunction,
    lora_qkv,
)
