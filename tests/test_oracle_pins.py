"""Pins of the CPU oracle to what the pages and the mathematics fix (no GPU).

Each test is chosen so that a plausible mistake in the oracle (a dropped term, a wrong sign or index, a
transposed operand, a wrong GQA mapping or mask alignment) fails at least one of them; the mutation tests at the
end plant such mistakes in copies of the oracle and check that the pins catch them.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import paged as opaged
from workloads import build_decode, build_prefill, make_config

# ------------------------------------------------------------------------------------------ slot / block arithmetic


def test_slot_formula_worked_example(golden):
    g = golden["slot_formula"]
    assert oracle.slot_of(g["block_id"], g["block_size"], g["loc"]) == g["slot"]


def test_prepare_prefill_example(golden):
    g = golden["prepare_prefill"]
    seqs = g["sequences"]
    table = np.full((len(seqs), 1), -1, np.int32)
    for i, s in enumerate(seqs):
        table[i, :len(s["block_table"])] = s["block_table"]
    n_new = [s["new_tokens"] for s in seqs]
    meta = oracle.build_metadata(table, [0] * len(seqs), n_new, g["block_size"])
    assert meta["positions"].tolist() == g["positions"]
    assert meta["cu_seqlens_q"].tolist() == g["cu_seqlens_q"]
    assert meta["slot_mapping"].tolist() == g["slot_mapping"]
    assert meta["total_q"] == g["cu_seqlens_q"][-1]


def test_block_arithmetic_example(golden):
    g = golden["block_arithmetic"]
    bs, n = g["block_size"], g["num_tokens"]
    assert oracle.num_blocks(n, bs) == g["num_blocks"]
    assert oracle.last_block_num_tokens(n, bs) == g["tokens_per_block"][-1]
    tokens = list(range(n))
    per_block = [len(tokens[oracle.block_token_slice(i, n, bs)]) for i in range(g["num_blocks"])]
    assert per_block == g["tokens_per_block"]
    assert len(tokens[oracle.block_token_slice(2, n, bs)]) == g["block2_len"]
    with pytest.raises(IndexError):
        oracle.block_token_slice(3, n, bs)
    # the get_slots listing covers exactly n slots, block by block
    slots = oracle.get_slots(g["block_table"], bs, n)
    assert len(slots) == n
    assert slots[0] == 5 * bs and slots[255] == 5 * bs + 255 and slots[256] == 9 * bs and slots[-1] == 12 * bs + 87


@pytest.mark.parametrize("bs", [1, 4, 16, 256])
def test_block_count_boundaries(bs):
    for k in range(1, 5):
        n = k * bs  # an exactly full last block holds bs tokens, not 0
        assert oracle.num_blocks(n, bs) == k
        assert oracle.last_block_num_tokens(n, bs) == bs
        assert oracle.num_blocks(n + 1, bs) == k + 1
        assert oracle.last_block_num_tokens(n + 1, bs) == 1
    assert oracle.num_blocks(0, bs) == 0


def test_chunked_counters_example(golden):
    g = golden["chunked_counters"]
    bs, table = g["block_size"], np.array([g["block_table"]], np.int32)
    all_slots = oracle.get_slots(g["block_table"], bs, g["prompt"])
    for ch in g["chunks"]:
        meta = oracle.build_metadata(table, [ch["num_cached"]], [ch["num_scheduled"]], bs)
        assert meta["context_lens"].tolist() == [ch["cached_after"]]
        assert meta["cu_seqlens_k"].tolist() == [0, ch["cached_after"]]
        assert meta["positions"].tolist() == list(range(ch["num_cached"], ch["cached_after"]))
        # the per-token slot rule and the block-range listing agree on every slot of the chunk
        assert meta["slot_mapping"].tolist() == all_slots[ch["num_cached"]:ch["cached_after"]]
    # after the last chunk one generated token is appended: its decode step writes position 600
    meta = oracle.build_metadata(table, [g["prompt"]], [1], bs)
    assert meta["context_lens"].tolist() == [g["num_tokens_after_first_generated"]]


def test_pool_picture(golden):
    g = golden["pool_picture"]
    slots = oracle.get_slots(list(range(g["num_blocks"])), g["block_size"], g["max_tokens"])
    assert slots == list(range(g["num_blocks"] * g["block_size"]))


@pytest.mark.parametrize("bs", [1, 3, 4, 16, 256])
def test_get_slots_matches_per_token_rule(bs):
    rng = np.random.default_rng(bs)
    for n in [1, bs - 1 if bs > 1 else 1, bs, bs + 1, 3 * bs + 2, 700]:
        ids = rng.permutation(1000)[:oracle.num_blocks(n, bs)].tolist()
        meta = oracle.build_metadata(np.array([ids], np.int32), [0], [n], bs)
        assert meta["slot_mapping"].tolist() == oracle.get_slots(ids, bs, n)
        # every slot is unique and lies inside one of the sequence's blocks
        s = meta["slot_mapping"]
        assert len(set(s.tolist())) == n
        assert set((s // bs).tolist()) <= set(ids)


# ------------------------------------------------------------------------------------------ store


def test_store_writes_exactly_one_slot():
    """A token stored at slot 102 of a bs=4 pool changes exactly bytes [102*row, 103*row) of the flat pool."""
    nb, bs, Hkv, D = 32, 4, 2, 16
    rng = np.random.default_rng(0)
    kc = rng.standard_normal((nb, bs, Hkv, D)).astype(np.float32)
    vc = rng.standard_normal((nb, bs, Hkv, D)).astype(np.float32)
    k0, v0 = kc.copy(), vc.copy()
    k = rng.standard_normal((3, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((3, Hkv, D)).astype(np.float32)
    oracle.store_kvcache(kc, vc, k, v, np.array([-1, 102, -1], np.int32))
    row = Hkv * D * 4
    kb, k0b = kc.view(np.uint8).reshape(-1), k0.view(np.uint8).reshape(-1)
    changed = np.flatnonzero(kb != k0b)
    assert changed.min() >= 102 * row and changed.max() < 103 * row
    assert np.array_equal(kc[25, 2], k[1]) and np.array_equal(vc[25, 2], v[1])
    kc[25, 2], vc[25, 2] = k0[25, 2], v0[25, 2]
    assert np.array_equal(kc, k0) and np.array_equal(vc, v0)


def test_store_bf16_is_bit_copy():
    nb, bs, Hkv, D = 8, 4, 2, 8
    rng = np.random.default_rng(1)
    kc = rng.integers(0, 65536, (nb, bs, Hkv, D), dtype=np.uint16)
    vc = kc.copy()
    k = rng.integers(0, 65536, (5, Hkv, D), dtype=np.uint16)  # includes NaN/Inf bit patterns
    slots = np.array([0, 31, 7, 8, 20], np.int32)
    oracle.store_kvcache(kc, vc, k, k, slots)
    flat = kc.reshape(nb * bs, Hkv, D)
    for i, s in enumerate(slots):
        assert np.array_equal(flat[s], k[i])


# ------------------------------------------------------------------------------------------ attention: brute force


def _brute_force(q, K, V, scale, q_pos):
    """Scalar loops with math.exp, float64: the definition with nothing vectorised."""
    n, Hq, D = q.shape
    k_len, Hkv, _ = K.shape
    G = Hq // Hkv
    out = np.zeros((n, Hq, D))
    for r in range(n):
        for h in range(Hq):
            g = h // G
            vis = [c for c in range(k_len) if c <= q_pos[r]]
            s = [scale * sum(float(q[r, h, d]) * float(K[c, g, d]) for d in range(D)) for c in vis]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = sum(w)
            for d in range(D):
                out[r, h, d] = sum(w[i] * float(V[c, g, d]) for i, c in enumerate(vis)) / z
    return out


def test_tiny_config_against_brute_force():
    wl = make_config("tiny")
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    for step in wl.steps:
        meta, out = oracle.run_step(step, kc, vc, wl.block_size, wl.scale, wl.dtype)
        # brute force from a gather done with get_slots (the pages' listing), not with gather_kv
        kf = kc.reshape(-1, wl.num_kv_heads, wl.head_dim)
        vf = vc.reshape(-1, wl.num_kv_heads, wl.head_dim)
        for s in range(step.batch):
            k_len = int(meta["context_lens"][s])
            ids = [int(x) for x in step.block_table[s] if x >= 0][:oracle.num_blocks(k_len, wl.block_size)]
            sl = oracle.get_slots(ids, wl.block_size, k_len)
            q0, q1 = int(meta["cu_seqlens_q"][s]), int(meta["cu_seqlens_q"][s + 1])
            ref = _brute_force(step.q[q0:q1].astype(np.float64), kf[sl].astype(np.float64),
                               vf[sl].astype(np.float64), wl.scale, meta["positions"][q0:q1])
            np.testing.assert_allclose(out[q0:q1], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_tiny_shapes_against_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    Hkv = int(rng.integers(1, 3))
    G = int(rng.integers(1, 4))
    D = int(rng.integers(2, 6))
    bs = int(rng.integers(1, 5))
    k_lens = rng.integers(1, 9, size=2)
    cached = np.array([int(rng.integers(0, n)) for n in k_lens])
    wl = build_prefill("t", seed, Hkv * G, Hkv, D, bs, "f32", k_lens, cached, num_blocks=40, scale=0.7)
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    meta, out = oracle.run_step(wl.steps[0], kc, vc, bs, wl.scale, "f32")
    step = wl.steps[0]
    for s in range(2):
        k_len = int(meta["context_lens"][s])
        K = oracle.gather_kv(kc, step.block_table[s], k_len).astype(np.float64)
        V = oracle.gather_kv(vc, step.block_table[s], k_len).astype(np.float64)
        q0, q1 = meta["cu_seqlens_q"][s], meta["cu_seqlens_q"][s + 1]
        ref = _brute_force(step.q[q0:q1].astype(np.float64), K, V, wl.scale, meta["positions"][q0:q1])
        np.testing.assert_allclose(out[q0:q1], ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------------------ closed forms


def test_single_key_returns_that_value():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 4, 8))
    K = rng.standard_normal((1, 2, 8))
    V = rng.standard_normal((1, 2, 8))
    out = oracle.attention_dense(q, K, V, 0.3, np.array([0]))
    assert np.array_equal(out[0, :2], np.repeat(V[0, :1], 2, axis=0))
    assert np.array_equal(out[0, 2:], np.repeat(V[0, 1:], 2, axis=0))


def test_zero_query_gives_causal_prefix_mean():
    rng = np.random.default_rng(4)
    k_len, q_len = 11, 5
    K = rng.standard_normal((k_len, 2, 6))
    V = rng.standard_normal((k_len, 2, 6))
    q = np.zeros((q_len, 4, 6))
    pos = np.arange(k_len - q_len, k_len)
    out = oracle.attention_dense(q, K, V, 1.0, pos)
    for r in range(q_len):
        for h in range(4):
            np.testing.assert_allclose(out[r, h], V[:pos[r] + 1, h // 2].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_dominant_key_selects_its_value():
    """One key aligned with the query and far larger than the rest: the output is that key's value."""
    rng = np.random.default_rng(5)
    D = 8
    K = rng.standard_normal((6, 1, D)) * 0.01
    K[2, 0] = np.ones(D) * 10
    V = rng.standard_normal((6, 1, D))
    q = np.ones((1, 1, D)) * 10
    out = oracle.attention_dense(q, K, V, 1.0, np.array([5]))
    np.testing.assert_allclose(out[0, 0], V[2, 0], atol=1e-12)
    out = oracle.attention_dense(q, K, V, 1.0, np.array([1]))  # key 2 is in the future: not selected
    assert not np.allclose(out[0, 0], V[2, 0], atol=1e-3)


# ------------------------------------------------------------------------------------------ library special case


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (8, 2), (6, 3), (4, 4)])
def test_contiguous_single_sequence_matches_torch_sdpa(Hq, Hkv):
    """Contiguous blocks, one sequence, q_len == k_len: torch's causal SDPA (GQA via enable_gqa) in float64."""
    rng = np.random.default_rng(Hq * 10 + Hkv)
    n, D, bs = 13, 16, 4
    wl = build_prefill("sdpa", 7, Hq, Hkv, D, bs, "f32", [n], [0], scale=0.37)
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    _, out = oracle.run_step(wl.steps[0], kc, vc, bs, wl.scale, "f32")
    step = wl.steps[0]
    q = torch.from_numpy(step.q.astype(np.float64)).transpose(0, 1)[None]  # [1, Hq, n, D]
    k = torch.from_numpy(step.k.astype(np.float64)).transpose(0, 1)[None]
    v = torch.from_numpy(step.v.astype(np.float64)).transpose(0, 1)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=0.37, enable_gqa=True)
    np.testing.assert_allclose(out, ref[0].transpose(0, 1).numpy(), rtol=1e-11, atol=1e-12)
    del rng


def test_bf16_decoding_matches_torch():
    bits = np.arange(0, 65536, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite values only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(opaged.to_f64(bits, "bf16"), ref)


# ------------------------------------------------------------------------------------------ consistency properties


def test_chunked_rows_equal_unchunked_rows():
    """Rows p.. of a full causal prefill equal a chunked prefill whose first p tokens are cached (bottom-right)."""
    Hq, Hkv, D, bs, n = 4, 2, 8, 4, 19
    full = build_prefill("full", 11, Hq, Hkv, D, bs, "f32", [n], [0])
    kc, vc = full.k_cache.copy(), full.v_cache.copy()
    _, out_full = oracle.run_step(full.steps[0], kc, vc, bs, full.scale, "f32")
    for p in [1, 4, 7, 18]:
        step = full.steps[0]
        chunk = type(step)("prefill", step.block_table, np.array([p], np.int32), np.array([n - p], np.int32),
                           step.q[p:], step.k[p:], step.v[p:])
        kc2, vc2 = full.k_cache.copy(), full.v_cache.copy()
        oracle.store_kvcache(kc2, vc2, step.k[:p], step.v[:p], oracle.get_slots(
            step.block_table[0][:oracle.num_blocks(n, bs)], bs, n)[:p])
        _, out_chunk = oracle.run_step(chunk, kc2, vc2, bs, full.scale, "f32")
        np.testing.assert_allclose(out_chunk, out_full[p:], rtol=1e-13, atol=1e-14)


def test_decode_equals_last_prefill_row():
    Hq, Hkv, D, bs, n = 8, 2, 8, 4, 10
    full = build_prefill("full", 12, Hq, Hkv, D, bs, "f32", [n], [0])
    kc, vc = full.k_cache.copy(), full.v_cache.copy()
    _, out_full = oracle.run_step(full.steps[0], kc, vc, bs, full.scale, "f32")
    step = full.steps[0]
    dec = type(step)("decode", step.block_table, np.array([n - 1], np.int32), np.array([1], np.int32),
                     step.q[-1:], step.k[-1:], step.v[-1:])
    _, out_dec = oracle.run_step(dec, kc, vc, bs, full.scale, "f32")  # the cache already holds all n tokens
    np.testing.assert_allclose(out_dec[0], out_full[-1], rtol=1e-13, atol=1e-14)


def _relabel(wl, perm):
    """The same workload with physical block b renamed perm[b] (contents move with the id)."""
    kc = np.empty_like(wl.k_cache)
    vc = np.empty_like(wl.v_cache)
    kc[perm] = wl.k_cache
    vc[perm] = wl.v_cache
    steps = []
    for st in wl.steps:
        bt = np.where(st.block_table >= 0, perm[np.maximum(st.block_table, 0)], -1).astype(np.int32)
        steps.append(type(st)(st.kind, bt, st.num_cached, st.num_new, st.q, st.k, st.v))
    return kc, vc, steps


@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_physical_relabelling_invariance(kind):
    if kind == "prefill":
        wl = build_prefill("p", 13, 4, 2, 8, 4, "bf16", [9, 14, 5], [4, 0, 2], num_blocks=12)
    else:
        wl = build_decode("d", 14, 4, 2, 8, 4, "bf16", [9, 14, 5], num_blocks=12)
    perm = np.random.default_rng(1).permutation(wl.num_blocks)
    kc, vc, steps = _relabel(wl, perm)
    kc0, vc0 = wl.k_cache.copy(), wl.v_cache.copy()
    _, a = oracle.run_step(wl.steps[0], kc0, vc0, wl.block_size, wl.scale, "bf16")
    _, b = oracle.run_step(steps[0], kc, vc, wl.block_size, wl.scale, "bf16")
    assert np.array_equal(a, b)
    assert np.array_equal(kc[perm], kc0) and np.array_equal(vc[perm], vc0)


def test_unreferenced_slots_do_not_matter():
    """NaN everywhere outside a sequence's first k_len slots (and outside the new tokens' slots) changes nothing."""
    wl = build_decode("d", 15, 4, 2, 8, 4, "f32", [9, 6], num_blocks=10)
    step = wl.steps[0]
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    meta, ref = oracle.run_step(step, kc, vc, wl.block_size, wl.scale, "f32")
    keep = np.zeros(wl.num_blocks * wl.block_size, bool)
    for s in range(step.batch):
        k_len = int(meta["context_lens"][s])
        ids = step.block_table[s][:oracle.num_blocks(k_len, wl.block_size)]
        keep[oracle.get_slots(ids, wl.block_size, k_len)] = True
    kp, vp = wl.k_cache.copy(), wl.v_cache.copy()
    kp.reshape(-1, 2, 8)[~keep] = np.nan
    vp.reshape(-1, 2, 8)[~keep] = np.nan
    _, out = oracle.run_step(step, kp, vp, wl.block_size, wl.scale, "f32")
    assert np.array_equal(out, ref)


def test_scale_enters_as_a_logit_multiplier():
    """Scaling q by a and the softmax scale by 1/a leaves the output unchanged; scale 0 gives the prefix mean."""
    rng = np.random.default_rng(6)
    q = rng.standard_normal((3, 2, 4))
    K = rng.standard_normal((7, 1, 4))
    V = rng.standard_normal((7, 1, 4))
    pos = np.array([4, 5, 6])
    a = oracle.attention_dense(q, K, V, 0.5, pos)
    b = oracle.attention_dense(q * 4.0, K, V, 0.125, pos)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)
    z = oracle.attention_dense(q, K, V, 0.0, pos)
    np.testing.assert_allclose(z[2, 0], V[:7, 0].mean(axis=0), rtol=1e-13)


# ------------------------------------------------------------------------------------------ mutation checks


def _mutant_attention(kind):
    def fn(q, K, V, scale, q_pos):
        n, Hq, _ = q.shape
        k_len, Hkv, _ = K.shape
        G = Hq // Hkv
        out = np.empty(q.shape)
        cols = np.arange(k_len)[None, :]
        pos = np.asarray(q_pos)
        for h in range(Hq):
            g = h % Hkv if kind == "gqa" else h // G
            S = (q[:, h, :] @ K[:, g, :].T) * (1.0 if kind == "scale" else scale)
            if kind == "mask_topleft":
                hidden = cols > (pos - pos[0])[:, None]
            else:
                hidden = cols > pos[:, None]
            S[hidden] = -np.inf
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            out[:, h, :] = P @ (K if kind == "kv_swap" else V)[:, g, :]
        return out
    return fn


@pytest.mark.parametrize("kind", ["gqa", "scale", "mask_topleft", "kv_swap"])
def test_pins_catch_planted_mistakes(monkeypatch, kind):
    """A wrong GQA mapping, a dropped scale, a top-left causal mask or K used as V fails the pins above."""
    monkeypatch.setattr(opaged, "attention_dense", _mutant_attention(kind))
    failures = 0
    for test in (lambda: test_contiguous_single_sequence_matches_torch_sdpa(4, 2),
                 test_chunked_rows_equal_unchunked_rows,
                 test_zero_query_gives_causal_prefix_mean,
                 test_tiny_config_against_brute_force):
        try:
            test()
        except AssertionError:
            failures += 1
    assert failures >= 1
