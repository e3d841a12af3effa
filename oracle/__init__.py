"""CPU oracle for the paged-KV attention step -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this package. The product path
(the HIP library and its Python binding) never imports, calls or links it, and it imports nothing from them.

It is the plain definition of what the step computes, written out in NumPy float64:
  * the slot arithmetic and block-count rules printed on the pages (metadata.py);
  * store_kvcache as a scatter into the flat slot view of the pool, and the block-table gather (paged.py);
  * naive softmax(Q K^T * scale + causal mask) V per query head (paged.py);
  * the pre-attention step of the new tokens: q_norm/k_norm RMSNorm, rotary embedding by table lookup, and
    the store of the rotated K and of V (rope.py);
  * next-token sampling with temperature, softmax and Gumbel-max, with its Philox counter-based generator
    (sampler.py).
"""

from .metadata import (  # noqa: F401
    slot_of,
    num_blocks,
    last_block_num_tokens,
    block_token_slice,
    get_slots,
    build_metadata,
)
from .paged import (  # noqa: F401
    to_f64,
    store_kvcache,
    gather_kv,
    attention_dense,
    prefill_varlen,
    decode,
    run_step,
)
from .rope import (  # noqa: F401
    rms_norm,
    rope_rotate_half,
    norm_rope,
    round_to,
    norm_rope_store,
)
from .sampler import (  # noqa: F401
    philox4x32_10,
    uniforms,
    gumbel_scores,
    sample,
)
