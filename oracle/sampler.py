"""Sampling of the next token from each sequence's logits: temperature, softmax, Gumbel-max, in plain NumPy.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg, never by
the product path. It shares no code with the HIP library.

The sampler divides the logits by the sequence's temperature, takes the softmax and draws with the Gumbel-max
trick ("Nano-vLLM 架构详解" §2.4, the sampling stage: temperature, softmax and Gumbel max; "一个 prompt 的一生"
§4: lm_head -> logits -> Sampler (Gumbel-max) -> token ids). Gumbel-max: with g_i = -log(-log u_i) for
independent uniforms u_i, argmax_i (log p_i + g_i) is distributed as p; since log p_i = l_i / T - logsumexp(l / T)
and the second term is the same for every i, the token is argmax_i (l_i / T + g_i). A temperature of 0 (or
below) is read as greedy decoding (argmax_i l_i). Ties go to the lower index.

Random numbers: each side implements the same counter-based generator from its published definition, Philox4x32
with 10 rounds (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random numbers: as easy as 1, 2,
3", SC 2011): a 128-bit counter (x0, x1, x2, x3) and a 64-bit key (k0, k1); one round maps the counter to
(hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)) with M0 = 0xD2511F53, M1 = 0xCD9E8D57, and the key
is bumped by (0x9E3779B9, 0xBB67AE85) between rounds. Element i of row b at call offset o uses word i % 4 of the
block for counter (i // 4, b, o mod 2^32, o div 2^32) under key (seed mod 2^32, seed div 2^32), and the uniform
u = ((x >> 9) + 1/2) * 2^-23, which float32 holds exactly and which lies strictly inside (0, 1).
"""

from __future__ import annotations

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32 with 10 rounds on arrays of 32-bit counter words; returns the four output words (uint32)."""
    x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) & MASK32 for c in (c0, c1, c2, c3))
    ka, kb = np.uint64(k0 & MASK32), np.uint64(k1 & MASK32)
    m0, m1 = np.uint64(M0), np.uint64(M1)
    for r in range(10):
        if r:
            ka = (ka + np.uint64(W0)) & np.uint64(MASK32)
            kb = (kb + np.uint64(W1)) & np.uint64(MASK32)
        p0 = x0 * m0  # < 2^64: exact in uint64
        p1 = x2 * m1
        x0, x1, x2, x3 = ((p1 >> np.uint64(32)) ^ x1 ^ ka, p1 & np.uint64(MASK32),
                          (p0 >> np.uint64(32)) ^ x3 ^ kb, p0 & np.uint64(MASK32))
    return tuple(w.astype(np.uint32) for w in (x0, x1, x2, x3))


def uniforms(rows, vocab: int, seed: int, offset: int) -> np.ndarray:
    """The float32 uniforms u_i, i < vocab, of the given rows ([len(rows), vocab]; see the module docstring for
    the counter layout)."""
    rows = np.atleast_1d(np.asarray(rows, dtype=np.uint64))
    blocks = (vocab + 3) // 4
    c0 = np.broadcast_to(np.arange(blocks, dtype=np.uint64)[None, :], (rows.size, blocks))
    c1 = np.broadcast_to(rows[:, None], (rows.size, blocks))
    words = philox4x32_10(c0, c1, np.full(c0.shape, offset & MASK32), np.full(c0.shape, (offset >> 32) & MASK32),
                          seed & MASK32, (seed >> 32) & MASK32)
    x = np.stack(words, axis=2).reshape(rows.size, 4 * blocks)[:, :vocab]
    return ((x >> np.uint32(9)).astype(np.float32) + np.float32(0.5)) * np.float32(2.0 ** -23)


def gumbel_scores(logits: np.ndarray, temperatures, u: np.ndarray, dtype=np.float32) -> np.ndarray:
    """l_i / T + g_i with g_i = -log(-log u_i) per row ([B, V]), in the given precision: float32 takes the decision
    the way the kernel does, float64 gives the exact values. Rows with T <= 0 score the logits alone (greedy)."""
    l = np.asarray(logits, dtype=dtype)
    t = np.asarray(temperatures, dtype=np.float64).reshape(-1, 1)
    g = -np.log(-np.log(np.asarray(u, dtype=dtype)))
    with np.errstate(divide="ignore", invalid="ignore"):
        inv_t = (dtype(1.0) / t.astype(dtype)).astype(dtype)
        scores = l * inv_t + g
    return np.where(t <= 0.0, l, scores).astype(dtype)


def sample(logits: np.ndarray, temperatures, seed: int, offset: int, dtype=np.float32, rows=None):
    """Token ids [B] (first maximum: ties go to the lower index) and the scores they maximise ([B, V], in
    `dtype`). rows: the row index of each logits row in the counter (default 0 .. B-1)."""
    logits = np.atleast_2d(logits)
    B, V = logits.shape
    rows = np.arange(B) if rows is None else rows
    scores = gumbel_scores(logits, temperatures, uniforms(rows, V, seed, offset), dtype)
    return np.argmax(scores, axis=1).astype(np.int32), scores
