"""Seeded generators for the five named workloads and for the small parity cases.

Everything here is a random draw or a layout decision. The one integer rule used, "a sequence of n tokens holds
ceil(n / block_size) blocks", is how many ids the emulated block manager hands out; the oracle and the kernels
never read it from here, they recompute block positions from the lengths and the table themselves.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CONFIG_NAMES = (
    "tiny",               # 16 blocks, bs=4, Hq=4, Hkv=2, D=16, fp32: store, prefill, three decode steps
    "decode_qwen3_0p6b",  # Hq=16, Hkv=8, D=128, bf16, bs=256, B=64, ctx U[128, 4096], pool 4096 blocks
    "prefill_qwen3_8b",   # Hq=32, Hkv=8, D=128, bf16, bs=256, B=8, L U[256, 2048], 0-2 cached blocks
    "decode_qwen3_32b",   # Hq=64, Hkv=8, D=128, bf16, bs=256, B=256, ctx log-U[1024, 32768], 25% shared prefix
    "chunked_qwen3_8b",   # Hq=32, Hkv=8, D=128, bf16, bs=256, q=2048 over k=32768, 1% x8 outliers
)

_CHUNK_BLOCKS = 8  # pool blocks per independently seeded chunk (keeps generation parallel and reproducible)
_THREADS = max(1, min(16, os.cpu_count() or 1))


@dataclass
class Step:
    """One call of the attention step: store the new tokens' K/V, then attend.

    kind         "prefill" (varlen causal over the cache) or "decode" (one query token per sequence)
    block_table  int32 [B, max_blocks_per_seq]; row s lists sequence s's physical block ids, padded with -1
    num_cached   int32 [B]; tokens of sequence s whose K/V are already in the cache before this step
    num_new      int32 [B]; tokens of sequence s computed in this step (1 for decode)
    q            [T, Hq, D] query rows of the new tokens, sequences concatenated without padding
    k, v         [T, Hkv, D] the new tokens' keys and values
    Values are uint16 bf16 bit patterns for dtype "bf16", float32 for "f32".
    """

    kind: str
    block_table: np.ndarray
    num_cached: np.ndarray
    num_new: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray

    @property
    def batch(self) -> int:
        return int(self.num_new.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])


@dataclass
class Workload:
    """A cache pool plus a sequence of steps over it."""

    name: str
    seed: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    dtype: str          # "bf16" or "f32"
    scale: float        # softmax scale handed to the kernels
    k_cache: np.ndarray  # initial pool [num_blocks, block_size, Hkv, D]
    v_cache: np.ndarray
    steps: list = field(default_factory=list)
    notes: dict = field(default_factory=dict)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


# ----------------------------------------------------------------------------------------------- value drawing


def encode_values(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 draws -> stored representation (bf16 bits by round-to-nearest-even, or float32 unchanged)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype != "bf16":
        raise ValueError(f"unsupported dtype {dtype!r}")
    import torch  # CPU only: torch's float32 -> bfloat16 conversion rounds to nearest even

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _draw(rng: np.random.Generator, shape, dtype: str, outlier_p: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if outlier_p > 0.0:
        x[rng.random(shape) < outlier_p] *= np.float32(8.0)
    return encode_values(x, dtype)


def _fill_pool(seed: int, stream: int, shape, dtype: str, referenced: np.ndarray, outlier_p: float) -> np.ndarray:
    """Pool with N(0,1) values in every referenced block and zeros elsewhere.

    Chunk c (blocks [8c, 8c+8)) is drawn from its own generator seeded by (seed, stream, c), so the values do
    not depend on the thread count.
    """
    nblk = shape[0]
    out = np.zeros(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    nchunks = (nblk + _CHUNK_BLOCKS - 1) // _CHUNK_BLOCKS
    todo = [c for c in range(nchunks) if referenced[c * _CHUNK_BLOCKS:(c + 1) * _CHUNK_BLOCKS].any()]

    def work(c: int) -> None:
        lo, hi = c * _CHUNK_BLOCKS, min(nblk, (c + 1) * _CHUNK_BLOCKS)
        rng = np.random.default_rng([seed, stream, c])
        x = rng.standard_normal((hi - lo,) + tuple(shape[1:]), dtype=np.float32)
        if outlier_p > 0.0:
            x[rng.random(x.shape) < outlier_p] *= np.float32(8.0)
        x[~referenced[lo:hi]] = 0.0
        out[lo:hi] = encode_values(x, dtype)

    if len(todo) <= 2:
        for c in todo:
            work(c)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(work, todo))
    return out


def _blocks_for(n_tokens: int, block_size: int) -> int:
    # how many ids the emulated block manager gives a sequence of n tokens
    return -(-int(n_tokens) // int(block_size))


def _pad_tables(tables, width: int | None = None) -> np.ndarray:
    width = max((len(t) for t in tables), default=0) if width is None else width
    out = np.full((len(tables), max(width, 1)), -1, dtype=np.int32)
    for i, t in enumerate(tables):
        out[i, :len(t)] = t
    return out


# ----------------------------------------------------------------------------------------------- generic builders


def build_prefill(name, seed, num_heads, num_kv_heads, head_dim, block_size, dtype, k_lens, cached,
                  num_blocks=None, outlier_p=0.0, scale=None, table_width=None, fill=True,
                  allow_empty=False) -> Workload:
    """One varlen prefill step: sequence s has k_lens[s] tokens, of which cached[s] are already in the cache.

    Physical ids are consecutive slices of a seeded permutation of the pool (random, distinct). With
    allow_empty, a sequence may have no new token (cached[s] == k_lens[s]): it is in the batch but computes
    nothing.
    """
    rng = np.random.default_rng(seed)
    k_lens = np.asarray(k_lens, dtype=np.int64)
    cached = np.asarray(cached, dtype=np.int64)
    if np.any(cached < 0) or np.any(cached > k_lens) or (not allow_empty and np.any(cached == k_lens)):
        raise ValueError("need 0 <= cached < k_len for every sequence (<= with allow_empty)")
    need = [_blocks_for(n, block_size) for n in k_lens]
    if num_blocks is None:
        num_blocks = max(1, sum(need))
    if sum(need) > num_blocks:
        raise ValueError("pool too small")
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables, at = [], 0
    for nb in need:
        tables.append(perm[at:at + nb].tolist())
        at += nb
    referenced = np.zeros(num_blocks, dtype=bool)
    referenced[perm[:at]] = True
    shape = (num_blocks, block_size, num_kv_heads, head_dim)
    kc = _fill_pool(seed, 1, shape, dtype, referenced, outlier_p) if fill else None
    vc = _fill_pool(seed, 2, shape, dtype, referenced, outlier_p) if fill else None
    num_new = (k_lens - cached).astype(np.int32)
    T = int(num_new.sum())
    vr = np.random.default_rng([seed, 3])
    step = Step(
        kind="prefill",
        block_table=_pad_tables(tables, table_width),
        num_cached=cached.astype(np.int32),
        num_new=num_new,
        q=_draw(vr, (T, num_heads, head_dim), dtype, outlier_p),
        k=_draw(vr, (T, num_kv_heads, head_dim), dtype, outlier_p),
        v=_draw(vr, (T, num_kv_heads, head_dim), dtype, outlier_p),
    )
    return Workload(name, seed, num_heads, num_kv_heads, head_dim, block_size, num_blocks, dtype,
                    float(scale if scale is not None else 1.0 / math.sqrt(head_dim)), kc, vc, [step])


def build_decode(name, seed, num_heads, num_kv_heads, head_dim, block_size, dtype, ctx_lens,
                 num_blocks=None, shared=None, outlier_p=0.0, scale=None, table_width=None, fill=True) -> Workload:
    """One decode step: sequence s has ctx_lens[s] tokens counting the new one, ctx_lens[s]-1 already cached.

    shared: optional list of (sharer, owner, n) meaning the sharer's first n blocks are the owner's blocks
    (prefix caching hands the same full blocks to both). Owners and sharers must hold more than n full blocks of
    context so that the new token never lands in a shared block.
    """
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    if np.any(ctx < 1):
        raise ValueError("every context holds at least the new token")
    need = [_blocks_for(n, block_size) for n in ctx]
    shared = list(shared or [])
    sharer_of = {s: (o, n) for s, o, n in shared}
    for s, o, n in shared:
        if s == o or s in {x[1] for x in shared} or o in sharer_of:
            raise ValueError("a sequence is either an owner or a sharer, never both")
        if ctx[s] <= n * block_size or ctx[o] <= n * block_size:
            raise ValueError("shared blocks must be full and must not receive the new token")
    distinct = sum(need) - sum(n for _, _, n in shared)
    if num_blocks is None:
        num_blocks = max(1, distinct)
    if distinct > num_blocks:
        raise ValueError("pool too small")
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = [None] * len(ctx)
    at = 0
    for s in range(len(ctx)):  # owners and plain sequences first, in order
        if s in sharer_of:
            continue
        tables[s] = perm[at:at + need[s]].tolist()
        at += need[s]
    for s in range(len(ctx)):  # then sharers: the owner's first n ids, then fresh ones
        if s not in sharer_of:
            continue
        o, n = sharer_of[s]
        own = need[s] - n
        tables[s] = tables[o][:n] + perm[at:at + own].tolist()
        at += own
    referenced = np.zeros(num_blocks, dtype=bool)
    referenced[perm[:at]] = True
    shape = (num_blocks, block_size, num_kv_heads, head_dim)
    kc = _fill_pool(seed, 1, shape, dtype, referenced, outlier_p) if fill else None
    vc = _fill_pool(seed, 2, shape, dtype, referenced, outlier_p) if fill else None
    B = len(ctx)
    vr = np.random.default_rng([seed, 3])
    step = Step(
        kind="decode",
        block_table=_pad_tables(tables, table_width),
        num_cached=(ctx - 1).astype(np.int32),
        num_new=np.ones(B, dtype=np.int32),
        q=_draw(vr, (B, num_heads, head_dim), dtype, outlier_p),
        k=_draw(vr, (B, num_kv_heads, head_dim), dtype, outlier_p),
        v=_draw(vr, (B, num_kv_heads, head_dim), dtype, outlier_p),
    )
    wl = Workload(name, seed, num_heads, num_kv_heads, head_dim, block_size, num_blocks, dtype,
                  float(scale if scale is not None else 1.0 / math.sqrt(head_dim)), kc, vc, [step])
    wl.notes["shared"] = shared
    return wl


# ----------------------------------------------------------------------------------------------- named configs


def _tiny(seed: int = 101, fill: bool = True) -> Workload:
    """16 blocks of 4 slots, 4 query heads over 2 KV heads, D=16, fp32; prompts of 7 and 6 tokens.

    Steps: prefill of both prompts (nothing cached), then three decode steps that each append one token per
    sequence; a sequence gets its next block when its new token's position is a multiple of the block size and
    its table is full (the block manager's append rule).
    """
    bs, nblk, Hq, Hkv, D = 4, 16, 4, 2, 16
    rng = np.random.default_rng(seed)
    perm = rng.permutation(nblk).astype(np.int32).tolist()
    free = list(perm)
    prompts = [7, 6]
    tables = []
    for n in prompts:
        nb = _blocks_for(n, bs)
        tables.append(free[:nb])
        del free[:nb]
    width = 3
    steps = []
    vr = np.random.default_rng([seed, 3])
    T = sum(prompts)
    steps.append(Step("prefill", _pad_tables(tables, width), np.zeros(2, np.int32), np.array(prompts, np.int32),
                      _draw(vr, (T, Hq, D), "f32", 0.0), _draw(vr, (T, Hkv, D), "f32", 0.0),
                      _draw(vr, (T, Hkv, D), "f32", 0.0)))
    lens = list(prompts)
    for _ in range(3):
        for s in range(2):
            pos = lens[s]
            if pos % bs == 0 and pos // bs == len(tables[s]):
                tables[s] = tables[s] + [free.pop(0)]
        steps.append(Step("decode", _pad_tables(tables, width), np.array(lens, np.int32), np.ones(2, np.int32),
                          _draw(vr, (2, Hq, D), "f32", 0.0), _draw(vr, (2, Hkv, D), "f32", 0.0),
                          _draw(vr, (2, Hkv, D), "f32", 0.0)))
        lens = [n + 1 for n in lens]
    referenced = np.zeros(nblk, dtype=bool)
    for t in tables:
        referenced[t] = True
    shape = (nblk, bs, Hkv, D)
    kc = _fill_pool(seed, 1, shape, "f32", referenced, 0.0)
    vc = _fill_pool(seed, 2, shape, "f32", referenced, 0.0)
    return Workload("tiny", seed, Hq, Hkv, D, bs, nblk, "f32", 1.0 / math.sqrt(D), kc, vc, steps)


def _decode_0p6b(seed: int = 102, fill: bool = True) -> Workload:
    rng = np.random.default_rng([seed, 0])
    ctx = rng.integers(128, 4096 + 1, size=64)
    return build_decode("decode_qwen3_0p6b", seed, 16, 8, 128, 256, "bf16", ctx, num_blocks=4096, table_width=16,
                        fill=fill)


def _prefill_8b(seed: int = 103, fill: bool = True) -> Workload:
    """B=8 prompts, L ~ U{256..2048}; c ~ U{0,1,2} cached whole blocks, clipped to (L-1)//256 so q_len >= 1.

    Both kinds of sequence are kept: if no sequence drew c = 0, sequence 0 gets c = 0; if none drew c > 0, the
    first sequence longer than one block gets min(2, (L-1)//256).
    """
    rng = np.random.default_rng([seed, 0])
    L = rng.integers(256, 2048 + 1, size=8)
    c = np.minimum(rng.integers(0, 3, size=8), (L - 1) // 256)
    if not np.any(c == 0):
        c[0] = 0
    if not np.any(c > 0):
        i = int(np.flatnonzero(L > 256)[0]) if np.any(L > 256) else 0
        c[i] = min(2, (int(L[i]) - 1) // 256)
    wl = build_prefill("prefill_qwen3_8b", seed, 32, 8, 128, 256, "bf16", L, 256 * c, num_blocks=1024,
                       table_width=8, fill=fill)
    wl.notes["cached_blocks"] = c.tolist()
    return wl


def _decode_32b(seed: int = 104, fill: bool = True) -> Workload:
    """B=256, ctx = round(exp(U[ln 1024, ln 32768])); 64 sharers reuse the first 4 blocks of 64 owners.

    Owners and sharers redraw their length until it exceeds 1024, so the 4 shared blocks are full and the new
    token of either sequence lands in a block of its own.
    """
    rng = np.random.default_rng([seed, 0])
    lo, hi = math.log(1024), math.log(32768)
    ctx = np.rint(np.exp(rng.uniform(lo, hi, size=256))).astype(np.int64)
    order = rng.permutation(256)
    owners, sharers = order[:64], order[64:128]
    for s in np.concatenate([owners, sharers]):
        while ctx[s] <= 1024:
            ctx[s] = int(np.rint(np.exp(rng.uniform(lo, hi))))
    shared = [(int(s), int(o), 4) for s, o in zip(sharers, owners)]
    return build_decode("decode_qwen3_32b", seed, 64, 8, 128, 256, "bf16", ctx, shared=shared, table_width=128,
                        fill=fill)


def _chunked_8b(seed: int = 105, fill: bool = True) -> Workload:
    return build_prefill("chunked_qwen3_8b", seed, 32, 8, 128, 256, "bf16", [32768], [30720], num_blocks=128,
                         outlier_p=0.01, table_width=128, fill=fill)


def _chunk256_8b(seed: int = 106, fill: bool = True) -> Workload:
    """A small chunk over a long prefix (chunked prefill at its smallest useful size): the chunked recipe with
    256 new rows after 32512 cached keys, so one sequence has 2 query tiles per head."""
    return build_prefill("chunk256_qwen3_8b", seed, 32, 8, 128, 256, "bf16", [32768], [32512], num_blocks=128,
                         outlier_p=0.01, table_width=128, fill=fill)


_BUILDERS = {
    "tiny": _tiny,
    "decode_qwen3_0p6b": _decode_0p6b,
    "prefill_qwen3_8b": _prefill_8b,
    "decode_qwen3_32b": _decode_32b,
    "chunked_qwen3_8b": _chunked_8b,
    "chunk256_qwen3_8b": _chunk256_8b,
}


def build_rope_inputs(seed: int, num_tokens: int, num_heads: int, num_kv_heads: int, head_dim: int, dtype: str,
                      max_position: int, base: float = 1.0e6, positions=None) -> dict:
    """Inputs of the pre-attention step of num_tokens new tokens: q [T, Hq, D], k, v [T, Hkv, D] ~ N(0, 1), the
    q_norm / k_norm weights [D] ~ N(1, 0.1), token positions (drawn below max_position unless given), and the
    rotary table [max_position, D] float32 a model precomputes: cos of position * base^(-2i/D) for i < D/2 in the
    first half of a row, the sin in the second half (base 1e6 as in Qwen3's published configuration; the pages
    name the table lookup but not its constants)."""
    rng = np.random.default_rng([seed, 7])
    if positions is None:
        positions = rng.integers(0, max_position, size=num_tokens)
    positions = np.asarray(positions, dtype=np.int32)
    inv_freq = base ** (-np.arange(0, head_dim, 2, dtype=np.float64) / head_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos_sin = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    return {
        "q": encode_values(rng.standard_normal((num_tokens, num_heads, head_dim)), dtype),
        "k": encode_values(rng.standard_normal((num_tokens, num_kv_heads, head_dim)), dtype),
        "v": encode_values(rng.standard_normal((num_tokens, num_kv_heads, head_dim)), dtype),
        "q_weight": encode_values(1.0 + 0.1 * rng.standard_normal(head_dim), dtype),
        "k_weight": encode_values(1.0 + 0.1 * rng.standard_normal(head_dim), dtype),
        "positions": positions,
        "cos_sin": cos_sin,
        "eps": 1e-6,
    }


_SEEDS = {"tiny": 101, "decode_qwen3_0p6b": 102, "prefill_qwen3_8b": 103, "decode_qwen3_32b": 104,
          "chunked_qwen3_8b": 105, "chunk256_qwen3_8b": 106}


def make_config(name: str, seed: int | None = None, fill: bool = True) -> Workload:
    """The named workload with its fixed seed (101..106), or another seed of the same recipe.

    fill=False skips drawing the pool (k_cache/v_cache are None); lengths, tables and Q/K/V are still drawn.
    """
    return _BUILDERS[name](_SEEDS[name] if seed is None else seed, fill=fill)
