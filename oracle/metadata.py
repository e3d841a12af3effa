"""Slot and block arithmetic of the paged KV cache, written out from the pages -- TEST INFRASTRUCTURE ONLY.

Passages followed:
  * slot = blockID * blockSize + loc, unique over the whole pool ("Nano-vLLM 架构详解" §1, Step2, the slot
    formula and its worked example 25*4+2 = 102);
  * a sequence of n tokens occupies ceil(n / block_size) blocks, the last one holding
    n - (num_blocks - 1) * block_size tokens, and logical block i covers tokens [i*bs, (i+1)*bs)
    ("Nano-vLLM 源码逐行解析 第2篇", sequence.py: num_blocks, last_block_num_tokens, block(i));
  * get_slots: the slots of a sequence's tokens, block by block ("Nano-vLLM 架构详解" §3.2, the KV cache write
    function), here built from the token range of each logical block and the slot formula;
  * prefill flattening: tokens of all sequences concatenated without padding, positions counted per sequence,
    cu_seqlens_q as prefix sums, slot_mapping[i] the slot of flattened token i ("一个 prompt 的一生" §3.3.2, the
    prepare_prefill example with block_size 4);
  * a scheduled chunk starts at num_cached_tokens ("Nano-vLLM 源码逐行解析 第2篇", sequence.py counter example).
"""

from __future__ import annotations

import numpy as np


def slot_of(block_id: int, block_size: int, loc: int) -> int:
    """Global slot of in-block offset `loc` of physical block `block_id`."""
    return int(block_id) * int(block_size) + int(loc)


def num_blocks(num_tokens: int, block_size: int) -> int:
    """Blocks needed for num_tokens tokens (rounded up)."""
    return (int(num_tokens) + int(block_size) - 1) // int(block_size)


def last_block_num_tokens(num_tokens: int, block_size: int) -> int:
    """Tokens held by the last block: total minus what the full blocks before it hold."""
    return int(num_tokens) - (num_blocks(num_tokens, block_size) - 1) * int(block_size)


def block_token_slice(i: int, num_tokens: int, block_size: int) -> slice:
    """Token index range of logical block i (clipped at the sequence end)."""
    if not 0 <= i < num_blocks(num_tokens, block_size):
        raise IndexError("logical block out of range")
    return slice(i * block_size, min((i + 1) * block_size, int(num_tokens)))


def get_slots(block_ids, block_size: int, seq_len: int) -> list:
    """Slots of positions 0..seq_len-1 of a sequence laid out over block_ids: each logical block i holds the tokens
    of block_token_slice(i, ...), and token t of it sits at offset t - i * block_size of physical block
    block_ids[i] (slot formula). The blocks a sequence needs are num_blocks(seq_len, ...)."""
    slots = []
    for i in range(num_blocks(seq_len, block_size)):
        toks = block_token_slice(i, seq_len, block_size)
        slots.extend(slot_of(block_ids[i], block_size, t - i * block_size) for t in range(toks.start, toks.stop))
    return slots


def build_metadata(block_table: np.ndarray, num_cached, num_new, block_size: int) -> dict:
    """Flattened per-token metadata for one step, one plain loop over sequences and tokens.

    Sequence s computes tokens at absolute positions num_cached[s] .. num_cached[s] + num_new[s] - 1; afterwards
    its K/V length is k_len = num_cached + num_new. Returns int32 arrays:
      positions [T], slot_mapping [T], cu_seqlens_q [B+1], cu_seqlens_k [B+1], context_lens [B] (= k_len),
    and the host scalars total_q, max_seqlen_q, max_seqlen_k.
    """
    B = len(num_new)
    positions, slots = [], []
    cu_q, cu_k, ctx = [0], [0], []
    for s in range(B):
        c, n = int(num_cached[s]), int(num_new[s])
        k_len = c + n
        for r in range(n):
            pos = c + r
            blk = int(block_table[s][pos // block_size])
            positions.append(pos)
            slots.append(slot_of(blk, block_size, pos % block_size))
        cu_q.append(cu_q[-1] + n)
        cu_k.append(cu_k[-1] + k_len)
        ctx.append(k_len)
    i32 = lambda a: np.asarray(a, dtype=np.int32)  # noqa: E731
    return {
        "positions": i32(positions),
        "slot_mapping": i32(slots),
        "cu_seqlens_q": i32(cu_q),
        "cu_seqlens_k": i32(cu_k),
        "context_lens": i32(ctx),
        "total_q": cu_q[-1],
        "max_seqlen_q": max((int(x) for x in num_new), default=0),
        "max_seqlen_k": max(ctx, default=0),
    }
