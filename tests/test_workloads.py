"""The seeded generators produce the workloads they claim to (no GPU, no values for the large pools)."""

import math

import numpy as np
import pytest

import oracle
from workloads import CONFIG_NAMES, build_decode, build_prefill, make_config


def _valid_tables(step, block_size, allow_shared=0):
    """Every sequence has at least ceil(k_len/bs) real ids; ids are distinct across sequences up to sharing."""
    k_len = step.num_cached + step.num_new
    used = []
    for s in range(step.batch):
        nb = oracle.num_blocks(int(k_len[s]), block_size)
        row = step.block_table[s]
        assert np.all(row[:nb] >= 0)
        assert np.all(row[nb:] == -1)
        used.extend(row[:nb].tolist())
    assert len(used) - len(set(used)) == allow_shared
    return used


def test_tiny_recipe():
    wl = make_config("tiny")
    assert (wl.num_blocks, wl.block_size, wl.num_heads, wl.num_kv_heads, wl.head_dim) == (16, 4, 4, 2, 16)
    assert wl.dtype == "f32" and wl.scale == 0.25
    assert [s.kind for s in wl.steps] == ["prefill", "decode", "decode", "decode"]
    pre = wl.steps[0]
    assert pre.num_new.tolist() == [7, 6] and pre.num_cached.tolist() == [0, 0]
    for i, st in enumerate(wl.steps[1:], start=1):
        assert st.num_cached.tolist() == [7 + i - 1, 6 + i - 1] and st.num_new.tolist() == [1, 1]
        _valid_tables(st, 4)
    # a sequence gets a new block exactly when its new token opens one: A at decode 2 (pos 8), B at decode 3
    nblocks = [[int((st.block_table[s] >= 0).sum()) for s in range(2)] for st in wl.steps]
    assert nblocks == [[2, 2], [2, 2], [3, 2], [3, 3]]
    # earlier blocks never move
    for a, b in zip(wl.steps, wl.steps[1:]):
        for s in range(2):
            na = int((a.block_table[s] >= 0).sum())
            assert np.array_equal(a.block_table[s][:na], b.block_table[s][:na])


def test_decode_0p6b_recipe():
    wl = make_config("decode_qwen3_0p6b", fill=False)
    st = wl.steps[0]
    ctx = st.num_cached + 1
    assert st.batch == 64 and ctx.min() >= 128 and ctx.max() <= 4096
    assert st.q.shape == (64, 16, 128) and st.k.shape == (64, 8, 128) and st.q.dtype == np.uint16
    assert wl.num_blocks == 4096 and st.block_table.shape == (64, 16)
    _valid_tables(st, 256)
    assert wl.scale == pytest.approx(1 / math.sqrt(128))


def test_prefill_8b_recipe():
    wl = make_config("prefill_qwen3_8b", fill=False)
    st = wl.steps[0]
    L = st.num_cached + st.num_new
    assert st.batch == 8 and L.min() >= 256 and L.max() <= 2048 and L.sum() <= 16384
    c = st.num_cached // 256
    assert np.all(st.num_cached % 256 == 0) and np.all(c <= 2) and np.all(st.num_new >= 1)
    assert np.any(c == 0) and np.any(c > 0)
    assert np.all((st.num_new < L) == (c > 0))
    _valid_tables(st, 256)


def test_decode_32b_recipe():
    wl = make_config("decode_qwen3_32b", fill=False)
    st = wl.steps[0]
    ctx = st.num_cached + 1
    assert st.batch == 256 and ctx.min() >= 1024 and ctx.max() <= 32768
    shared = wl.notes["shared"]
    assert len(shared) == 64
    assert len({s for s, _, _ in shared} | {o for _, o, _ in shared}) == 128
    for s, o, n in shared:
        assert n == 4 and ctx[s] > 1024 and ctx[o] > 1024
        assert np.array_equal(st.block_table[s][:4], st.block_table[o][:4])
    used = _valid_tables(st, 256, allow_shared=64 * 4)
    assert wl.num_blocks == len(set(used))
    # element offsets of the K pool exceed 2^31: 64-bit addressing is exercised
    assert wl.num_blocks * 256 * 8 * 128 > 2 ** 31


def test_chunked_8b_recipe():
    wl = make_config("chunked_qwen3_8b", fill=False)
    st = wl.steps[0]
    assert st.num_cached.tolist() == [30720] and st.num_new.tolist() == [2048]
    assert sorted(st.block_table[0].tolist()) == list(range(128))
    x = st.q.astype(np.uint32) << 16
    vals = x.view(np.float32)
    assert np.mean(np.abs(vals) > 5.0) > 0.003  # the x8 outliers are there


def test_reproducible_and_seed_sensitive():
    a = build_prefill("a", 5, 4, 2, 8, 4, "bf16", [9, 5], [4, 0], num_blocks=9)
    b = build_prefill("a", 5, 4, 2, 8, 4, "bf16", [9, 5], [4, 0], num_blocks=9)
    c = build_prefill("a", 6, 4, 2, 8, 4, "bf16", [9, 5], [4, 0], num_blocks=9)
    assert np.array_equal(a.k_cache, b.k_cache) and np.array_equal(a.steps[0].q, b.steps[0].q)
    assert not np.array_equal(a.k_cache, c.k_cache)


def test_unreferenced_blocks_are_zero():
    wl = build_decode("d", 3, 4, 2, 8, 4, "f32", [5, 3], num_blocks=10)
    st = wl.steps[0]
    ref = set(st.block_table[st.block_table >= 0].tolist())
    for b in range(10):
        assert (np.any(wl.k_cache[b] != 0)) == (b in ref)


@pytest.mark.parametrize("name", CONFIG_NAMES)
def test_all_configs_build_tables(name):
    wl = make_config(name, fill=False)
    for st in wl.steps:
        assert st.block_table.dtype == np.int32 and st.num_new.dtype == np.int32
        assert st.q.shape[0] == int(st.num_new.sum())
