"""Seeded synthetic inputs for the paged-KV attention step.

This package only draws random numbers and lays them out the way an inference engine's block manager and
scheduler would hand them to the attention layer: sequence lengths, how many tokens of each sequence already
have K/V in the cache, the physical block ids given to each sequence, and the Q/K/V values. It computes none of
the method's arithmetic: no slot addresses, no prefix sums, no masks, no attention, no normalisation or
rotation (the rotary table itself is a model constant and is drawn here as an input). The CPU oracle and the HIP
path each derive those themselves from what is drawn here. Both read these arrays; neither shares code through
this package.

Source of the shapes: the cache pool is `[num_blocks, block_size, num_kv_heads, head_dim]` per layer and per K/V
("一个 prompt 的一生" §2.2.3; "Nano-vLLM 架构详解" §3.2, Attention 运算), a block table maps logical to physical
blocks ("Nano-vLLM 架构详解" §1 Step2), and a sequence continues at `num_cached_tokens` when a prefix is cached or a
prompt is chunked ("Nano-vLLM 源码逐行解析 第2篇", sequence.py counter example).
"""

from .gen import (  # noqa: F401
    Step,
    Workload,
    CONFIG_NAMES,
    make_config,
    build_prefill,
    build_decode,
    encode_values,
    build_rope_inputs,
)
