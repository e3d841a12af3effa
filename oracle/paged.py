"""store_kvcache, the block-table gather and causal GQA attention, in NumPy float64 -- TEST INFRASTRUCTURE ONLY.

Passages followed:
  * the pool of one layer is [num_blocks, block_size, num_kv_heads, head_dim], contiguous in (block, offset), so
    a slot indexes a flat [num_blocks*block_size, Hkv, D] view of it ("一个 prompt 的一生" §2.2.3; the Attention
    section of "Nano-vLLM 架构详解" §3.2 for the KV-cache and block_tables formats);
  * store_kvcache writes each new token's K and V at slot_mapping[i]; the write itself knows nothing about
    pages ("一个 prompt 的一生" §4 summary; "Nano-vLLM 架构详解" §3.2, the KV cache write function);
  * the attention layer first writes the cache, then calls the prefill or decode attention over it
    ("一个 prompt 的一生" §3.3.2 / §4; "Nano-vLLM 架构详解" §2.4 Attention stage);
  * block_table[i] is the physical block of logical block i, like a page table ("Nano-vLLM 源码逐行解析 第2篇",
    sequence.py), so the K/V of a sequence is its blocks concatenated in table order, cut to its length.

Readings where the pages are silent (each is listed in the design notes):
  * query head h reads KV head h // (Hq / Hkv) (contiguous GQA groups);
  * a query at absolute position pos sees keys 0..pos; the q_len new tokens of a sequence with k_len keys sit
    at positions k_len - q_len .. k_len - 1 (chunks continue at num_cached_tokens);
  * slot < 0 means "do not write".
"""

from __future__ import annotations

import numpy as np

from .metadata import build_metadata, num_blocks


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64. bf16 bits are the upper half of an IEEE float32."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float64)
    raise ValueError(f"unsupported dtype {dtype!r}")


def store_kvcache(k_cache: np.ndarray, v_cache: np.ndarray, k: np.ndarray, v: np.ndarray,
                  slot_mapping: np.ndarray) -> None:
    """In place: flat_cache[slot_mapping[i]] = new[i] for every token i with a non-negative slot (a bit copy)."""
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    kf = k_cache.reshape(nb * bs, -1)
    vf = v_cache.reshape(nb * bs, -1)
    T = k.shape[0]
    for i in range(T):
        slot = int(slot_mapping[i])
        if slot < 0:
            continue
        kf[slot] = k[i].reshape(-1)
        vf[slot] = v[i].reshape(-1)


def gather_kv(cache: np.ndarray, table_row, k_len: int) -> np.ndarray:
    """Contiguous [k_len, Hkv, D] for one sequence: its blocks in table order, first k_len rows."""
    bs = cache.shape[1]
    nb = num_blocks(k_len, bs)
    blocks = [cache[int(table_row[j])] for j in range(nb)]
    return np.concatenate(blocks, axis=0)[:k_len]


def attention_dense(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, q_pos: np.ndarray) -> np.ndarray:
    """softmax(q K^T * scale, keys after each query's position masked) V, per query head, in float64.

    q [n, Hq, D]; K, V [k_len, Hkv, D]; q_pos[r] is the absolute position of query row r. Query head h uses KV
    head h // (Hq // Hkv).
    """
    n, Hq, _ = q.shape
    k_len, Hkv, _ = K.shape
    G = Hq // Hkv
    out = np.empty(q.shape, dtype=np.float64)
    cols = np.arange(k_len)[None, :]
    hidden = cols > np.asarray(q_pos)[:, None]  # [n, k_len]
    for h in range(Hq):
        g = h // G
        S = (q[:, h, :] @ K[:, g, :].T) * scale
        S[hidden] = -np.inf
        S = S - S.max(axis=1, keepdims=True)
        P = np.exp(S)
        P /= P.sum(axis=1, keepdims=True)
        out[:, h, :] = P @ V[:, g, :]
    return out


def prefill_varlen(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, block_table, scale, dtype,
                   seqs=None, rows=None) -> np.ndarray:
    """Causal varlen attention over the paged cache; rows not computed are NaN.

    seqs: iterable of sequence indices to compute (default all); rows: optional {s: row indices within the
    sequence} to compute only some query rows of s.
    """
    total_q, Hq, D = q.shape
    out = np.full((total_q, Hq, D), np.nan)
    B = len(cu_seqlens_q) - 1
    for s in (range(B) if seqs is None else seqs):
        q0, q1 = int(cu_seqlens_q[s]), int(cu_seqlens_q[s + 1])
        k_len = int(cu_seqlens_k[s + 1]) - int(cu_seqlens_k[s])
        q_len = q1 - q0
        if q_len == 0:
            continue
        r = np.arange(q_len) if rows is None or s not in rows else np.asarray(rows[s])
        K = to_f64(gather_kv(k_cache, block_table[s], k_len), dtype)
        V = to_f64(gather_kv(v_cache, block_table[s], k_len), dtype)
        qs = to_f64(q[q0 + r], dtype)
        out[q0 + r] = attention_dense(qs, K, V, scale, (k_len - q_len) + r)
    return out


def decode(q, k_cache, v_cache, context_lens, block_table, scale, dtype, seqs=None) -> np.ndarray:
    """One query per sequence, at position context_lens[s]-1, over all context_lens[s] keys."""
    B, Hq, D = q.shape
    out = np.full((B, Hq, D), np.nan)
    for s in (range(B) if seqs is None else seqs):
        k_len = int(context_lens[s])
        K = to_f64(gather_kv(k_cache, block_table[s], k_len), dtype)
        V = to_f64(gather_kv(v_cache, block_table[s], k_len), dtype)
        out[s:s + 1] = attention_dense(to_f64(q[s:s + 1], dtype), K, V, scale, np.array([k_len - 1]))
    return out


def run_step(step, k_cache, v_cache, block_size, scale, dtype, seqs=None, rows=None):
    """Metadata, store (in place on the given pools), then attention for one workload step.

    Returns (metadata dict, float64 output [T, Hq, D]).
    """
    meta = build_metadata(step.block_table, step.num_cached, step.num_new, block_size)
    store_kvcache(k_cache, v_cache, step.k, step.v, meta["slot_mapping"])
    if step.kind == "prefill":
        out = prefill_varlen(step.q, k_cache, v_cache, meta["cu_seqlens_q"], meta["cu_seqlens_k"],
                             step.block_table, scale, dtype, seqs=seqs, rows=rows)
    else:
        out = decode(step.q, k_cache, v_cache, meta["context_lens"], step.block_table, scale, dtype, seqs=seqs)
    return meta, out
