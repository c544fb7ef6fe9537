"""fp64 CPU oracle for the Gemma 3 attention-block forward.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The product path (``global_layers_amd``) never imports it, and this
package never imports the product path: the two share no code, no constants
and no helpers. Only the seeded input generators in ``workloads`` feed both.

Every function is a plain, slow, literal statement of what the study-note
pages define, in float64, with numpy matmuls as the only library primitive.
"""

from .gemma3_oracle import (  # noqa: F401
    K_MASK,
    RMS_EPS,
    LOCAL_SLIDING,
    GLOBAL,
    ATTENTION_PATTERN,
    layer_attn_type,
    layer_attn_types,
    rms_norm,
    rope,
    project_qkv,
    allowed_mask,
    attention_core,
    prefill,
    decode,
    prefill_cache,
    prefill_chunk,
    gelu_tanh,
    feed_forward,
    block_prefill,
    block_decode,
    stack_prefill,
    stack_prefill_cache,
    stack_decode,
    kv_cache_bytes,
)
