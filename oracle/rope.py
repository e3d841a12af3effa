"""Pre-attention path of a layer for the new tokens, plain float64 NumPy: RMSNorm of each head (q_norm, k_norm),
rotary position embedding by table lookup, then the store of K (after both) and V (as is) into the paged cache.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg, never by
the product path. It shares no code with the HIP library.

Order within a decoder layer: q_norm -> k_norm -> rope -> store_kvcache ("一个 prompt 的一生：nano-vllm 从起服务到吐出
token" §2.2.4, the operator list of one layer); RoPE is applied by looking up a precomputed table (same page
§3.3.2). The pages give neither formula nor constants, so these are readings, each pinned by
tests/test_oracle_rope.py:
  * RMSNorm over head_dim: y = x / sqrt(mean(x^2) + eps) * w, with a learned weight w[head_dim] shared by the
    heads, computed per (token, head).
  * Rotation pairs are the two halves of a head: (x[i], x[i + D/2]) is rotated by the angle of frequency i at
    the token's position ("rotate half"): x[i] cos - x[i+D/2] sin, x[i+D/2] cos + x[i] sin.
  * The table holds one row per position, cos of the D/2 angles in [:D/2] and their sin in [D/2:].
"""

from __future__ import annotations

import numpy as np

from .paged import store_kvcache, to_f64


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * w over the last axis (float64)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def rope_rotate_half(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate the pairs (x[i], x[i + D/2]) by the angles whose cos/sin are given ([..., D/2], broadcast)."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def norm_rope(x: np.ndarray, w: np.ndarray, eps: float, positions: np.ndarray, cos_sin: np.ndarray) -> np.ndarray:
    """x [T, H, D] -> RMSNorm per (token, head) with weight w, then rotation by the table row of each token's
    position. cos_sin [max_position, D] float32 (values used as given)."""
    d = x.shape[-1]
    rows = np.asarray(cos_sin, dtype=np.float64)[np.asarray(positions, dtype=np.int64)]  # [T, D]
    cos = rows[:, None, : d // 2]
    sin = rows[:, None, d // 2:]
    return rope_rotate_half(rms_norm(x, w, eps), cos, sin)


def round_to(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the cache dtype (bf16 round-to-nearest-even as uint16 bits, or float32)."""
    if dtype == "f32":
        return np.asarray(x64, dtype=np.float32)
    f = np.asarray(x64, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (f + 0x7FFF + ((f >> 16) & 1)) >> 16
    nan = np.isnan(np.asarray(x64, dtype=np.float32))
    r = np.where(nan, 0x7FC0, r)
    return r.astype(np.uint16)


def norm_rope_store(k, v, k_weight, eps, positions, cos_sin, k_cache, v_cache, slot_mapping, dtype: str,
                    q=None, q_weight=None):
    """The fused step on the host: K' = rope(k_norm(k)) stored at its slot (rounded to the cache dtype), V stored
    as is, and, if q is given, Q' = rope(q_norm(q)) returned in float64. k/v/q and weights are stored-dtype
    arrays (bf16 as uint16 bits). Returns (k_rot_f64, q_rot_f64 or None)."""
    k64 = to_f64(k, dtype)
    kw = to_f64(k_weight, dtype)
    k_rot = norm_rope(k64, kw, eps, positions, cos_sin)
    store_kvcache(k_cache, v_cache, round_to(k_rot, dtype), v, slot_mapping)
    q_rot = None
    if q is not None:
        q_rot = norm_rope(to_f64(q, dtype), to_f64(q_weight, dtype), eps, positions, cos_sin)
    return k_rot, q_rot
