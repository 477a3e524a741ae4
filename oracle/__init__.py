"""CPU oracle (test infrastructure only): see oracle/smol.py.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. The product library never does.
"""

from .smol import (  # noqa: F401
    Config,
    LayerWeights,
    ModelWeights,
    attention_sublayer,
    block_forward,
    decode_step,
    embed,
    gqa_attention,
    lm_head,
    mlp_sublayer,
    model_prefill,
    param_count,
    param_shapes,
    rms_norm,
    rope_inv_freq,
    rope_rotate,
    silu,
    softmax,
    swiglu_mlp,
)
